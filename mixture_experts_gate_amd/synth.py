"""Seeded synthetic inputs for the routed MoE expert layer.

This module only *makes inputs*: activations, router logits, gate weights and
expert-weight blobs in their storage format. It computes nothing the layer
computes (no decode of the weight format, no routing, no contraction), so the
CPU oracle and the GPU path can both consume its output without sharing any of
the layer's arithmetic.

Workloads (FreeToken pages, "Why Now" section on the winzheng.com page: a few
routed experts per token per layer, FP4-quantised expert pool held in host
memory; aimodeling.com/en page, "Reported Numbers": MXFP4 / NVFP4 / FP8 / BF16
weight formats) are stood in for by the five layer shapes in ``CONFIGS``.

Every stream is addressed by ``SeedSequence(seed, spawn_key=(stream, a, b))`` so
that any tensor can be regenerated independently of generation order.
"""
from __future__ import annotations

import dataclasses
import os

import numpy as np

# --------------------------------------------------------------------------
# Workload table
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    H: int            # hidden size
    E: int            # routed experts
    k: int            # experts per token
    I: int            # expert SwiGLU intermediate size
    fmt: str          # "bf16" | "mxfp4"
    n_shared: int     # always-on shared experts (unweighted add)
    logits: str       # "gate" | "uniform" | "gumbel_bias" | "zipf"
    Ts: tuple         # token counts the workload is run at
    weights: str      # weight recipe: "gauss_bf16" | "gauss_mxfp4" | "marginal_mxfp4"
    layers: int = 1
    seed: int = 0
    weight_seed: int | None = None   # draw expert weights from another workload's seed

    @property
    def wseed(self) -> int:
        return self.seed if self.weight_seed is None else self.weight_seed


CONFIGS = {
    1: LayerConfig("tiny", 256, 8, 2, 512, "bf16", 0, "gate", (16,), "gauss_bf16", seed=1),
    2: LayerConfig("decode", 2048, 128, 8, 768, "mxfp4", 0, "uniform", (1, 8, 32, 64),
                   "gauss_mxfp4", seed=2),
    # the prefill workload runs the decode workload's layer (same weights) at T=8192
    3: LayerConfig("prefill", 2048, 128, 8, 768, "mxfp4", 0, "gumbel_bias", (8192,),
                   "gauss_mxfp4", seed=3, weight_seed=2),
    4: LayerConfig("large_sparse", 4096, 256, 6, 2048, "mxfp4", 1, "zipf", (1, 64, 4096),
                   "marginal_mxfp4", seed=4),
    5: LayerConfig("stack43", 4096, 256, 6, 2048, "mxfp4", 1, "zipf", (1, 2, 4, 8, 16),
                   "marginal_mxfp4", layers=43, seed=5),
}

WEIGHT_SIGMA = 0.02
GATE_SIGMA = 0.02
ZIPF_S = 1.1
ZIPF_PHASE_STEPS = 256      # popularity re-permuted every this many steps
DEAD_EXPERT_BIAS = -30.0
BIAS_SCALE = 0.22

# stream ids for spawn keys
_S_X, _S_W, _S_GATE, _S_LOGITS, _S_PERM, _S_BIAS, _S_SHARED = range(7)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


# --------------------------------------------------------------------------
# Storage layout of one expert (layout only; no decoding here)
# --------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class BlobLayout:
    """Byte offsets inside one contiguous expert blob.

    MXFP4: [W13 codes (2I rows x H/2 bytes)][W13 scales (2I x H/32)]
           [W2 codes (H rows x I/2 bytes)][W2 scales (H x I/32)]
    BF16:  [W13 (2I x H bf16)][W2 (H x I bf16)]; scale sections are empty.
    Rows 0..I-1 of W13 are the gate projection, rows I..2I-1 the up projection.
    In a code byte the low nibble is the even element along K.
    """
    fmt: str
    H: int
    I: int
    w13: int
    s13: int
    w2: int
    s2: int
    nbytes: int


def blob_layout(H: int, I: int, fmt: str) -> BlobLayout:
    if H % 32 or I % 32:
        raise ValueError("H and I must be multiples of 32")
    if fmt == "mxfp4":
        w13 = 0
        s13 = w13 + 2 * I * H // 2
        w2 = s13 + 2 * I * H // 32
        s2 = w2 + H * I // 2
        end = s2 + H * I // 32
    elif fmt == "nvfp4":
        # codes, E4M3 block scales (one per 16), then a 16-byte field with
        # the matrix's fp32 scale
        w13 = 0
        s13 = w13 + 2 * I * H // 2
        w2 = s13 + 2 * I * H // 16 + 16
        s2 = w2 + H * I // 2
        end = s2 + H * I // 16 + 16
    elif fmt == "fp8":
        # one-byte E4M3 codes, then a 16-byte field with the matrix's fp32 scale
        w13 = 0
        s13 = w13 + 2 * I * H
        w2 = s13 + 16
        s2 = w2 + H * I
        end = s2 + 16
    elif fmt == "bf16":
        w13 = 0
        w2 = 2 * I * H * 2
        s13 = w2                  # empty scale section
        end = w2 + H * I * 2
        s2 = end                  # empty scale section
    else:
        raise ValueError(fmt)
    return BlobLayout(fmt, H, I, w13, s13, w2, s2, end)


# --------------------------------------------------------------------------
# Element encoders used to *produce* stored weights
# --------------------------------------------------------------------------

# |value| * 2 -> E2M1 magnitude code (OCP Microscaling v1.0 element grid
# 0, 0.5, 1, 1.5, 2, 3, 4, 6)
_MAG2_TO_CODE = np.full(13, 255, dtype=np.uint8)
for _c, _m2 in enumerate((0, 1, 2, 3, 4, 6, 8, 12)):
    _MAG2_TO_CODE[_m2] = _c


def encode_mxfp4(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Quantise fp32 rows [R][K] to MX-format FP4 (E2M1 codes, E8M0 block scales).

    Shared exponent per 32-element block along K: floor(log2(amax)) - 2 (the
    E2M1 maximum exponent), clamped to [-127, 127]; elements scaled by 2^-e,
    rounded to nearest even on the E2M1 grid, saturated at +-6.
    Returns (codes [R][K/2] uint8 with the even element in the low nibble,
    scales [R][K/32] uint8 E8M0).
    """
    w = np.asarray(w, dtype=np.float32)
    R, K = w.shape
    blocks = w.reshape(R, K // 32, 32)
    amax = np.abs(blocks).max(axis=2)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(amax)).astype(np.float64) - 2.0
    e = np.where(amax > 0, e, -127.0)
    e = np.clip(e, -127, 127).astype(np.int32)
    scales = (e + 127).astype(np.uint8)
    q = blocks / np.ldexp(np.float32(1.0), e)[:, :, None].astype(np.float32)
    a = np.abs(q)
    # round-to-nearest-even on the non-uniform grid, one binade band at a time
    r = np.where(a < 2.0, np.rint(a * 2.0) / 2.0,
                 np.where(a < 4.0, np.rint(a), np.rint(a / 2.0) * 2.0))
    r = np.minimum(r, 6.0)
    mag = _MAG2_TO_CODE[(r * 2.0).astype(np.int64)]
    assert (mag != 255).all()
    sign = (np.signbit(q) & (mag != 0)).astype(np.uint8) << 3
    codes = (mag | sign).reshape(R, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales


def _round_e2m1(q: np.ndarray) -> np.ndarray:
    """Values (already divided by their scale) -> E2M1 codes, round to nearest
    even on the grid 0, 0.5, 1, 1.5, 2, 3, 4, 6, saturating at 6."""
    a = np.abs(q)
    r = np.where(a < 2.0, np.rint(a * 2.0) / 2.0,
                 np.where(a < 4.0, np.rint(a), np.rint(a / 2.0) * 2.0))
    r = np.minimum(r, 6.0)
    mag = _MAG2_TO_CODE[(r * 2.0).astype(np.int64)]
    sign = (np.signbit(q) & (mag != 0)).astype(np.uint8) << 3
    return (mag | sign).astype(np.uint8)


def _to_e4m3(a: np.ndarray) -> np.ndarray:
    """fp32 -> E4M3 codes (torch's float8_e4m3fn conversion, round to nearest
    even; inputs are kept inside the finite range by the callers)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _from_e4m3(c: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(c, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float32).numpy()


def encode_nvfp4(w: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.float32]:
    """Quantise fp32 rows [R][K] to NVFP4: a per-matrix fp32 scale
    g = amax / (6 * 448), E4M3 block scales s = amax_block / (6 g) per 16
    elements along K, E2M1 codes of w / (s g) (round to nearest even, saturating).
    Returns (codes [R][K/2] with the even element in the low nibble, block
    scales [R][K/16] as E4M3 bytes, g)."""
    w = np.asarray(w, dtype=np.float32)
    R, K = w.shape
    amax = float(np.abs(w).max())
    g = np.float32(amax / (6.0 * 448.0)) if amax > 0 else np.float32(1.0)
    blocks = w.reshape(R, K // 16, 16)
    bmax = np.abs(blocks).max(axis=2)
    sc = _to_e4m3(np.minimum(bmax / (6.0 * g), 448.0).astype(np.float32))
    sv = _from_e4m3(sc).astype(np.float32) * g
    q = np.where(sv[:, :, None] > 0, blocks / np.where(sv > 0, sv, 1.0)[:, :, None], 0.0)
    codes = _round_e2m1(q.astype(np.float32)).reshape(R, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, sc.reshape(R, K // 16), g


def encode_fp8(w: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """Quantise fp32 rows [R][K] to E4M3 codes of w / g, g = amax / 448."""
    w = np.asarray(w, dtype=np.float32)
    amax = float(np.abs(w).max())
    g = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
    return _to_e4m3(np.clip(w / g, -448.0, 448.0)), g


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 bit patterns (torch's RNE conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------
# Expert weights
# --------------------------------------------------------------------------


def _gauss_mxfp4_blob(rng: np.random.Generator, H: int, I: int, sigma: float) -> np.ndarray:
    lay = blob_layout(H, I, "mxfp4")
    out = np.empty(lay.nbytes, dtype=np.uint8)
    w13 = rng.standard_normal((2 * I, H), dtype=np.float32) * np.float32(sigma)
    c13, s13 = encode_mxfp4(w13)
    del w13
    w2 = rng.standard_normal((H, I), dtype=np.float32) * np.float32(sigma)
    c2, s2 = encode_mxfp4(w2)
    out[lay.w13:lay.s13] = c13.reshape(-1)
    out[lay.s13:lay.w2] = s13.reshape(-1)
    out[lay.w2:lay.s2] = c2.reshape(-1)
    out[lay.s2:lay.nbytes] = s2.reshape(-1)
    return out


def _scale_field(g) -> np.ndarray:
    f = np.zeros(16, dtype=np.uint8)
    f[:4] = np.array([g], dtype=np.float32).view(np.uint8)
    return f


def _gauss_nvfp4_blob(rng: np.random.Generator, H: int, I: int, sigma: float) -> np.ndarray:
    lay = blob_layout(H, I, "nvfp4")
    out = np.empty(lay.nbytes, dtype=np.uint8)
    for (rows, cols, o_c, o_s, o_end) in ((2 * I, H, lay.w13, lay.s13, lay.w2),
                                          (H, I, lay.w2, lay.s2, lay.nbytes)):
        w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(sigma)
        c, sc, g = encode_nvfp4(w)
        out[o_c:o_s] = c.reshape(-1)
        out[o_s:o_s + rows * cols // 16] = sc.reshape(-1)
        out[o_s + rows * cols // 16:o_end] = _scale_field(g)
    return out


def _gauss_fp8_blob(rng: np.random.Generator, H: int, I: int, sigma: float) -> np.ndarray:
    lay = blob_layout(H, I, "fp8")
    out = np.empty(lay.nbytes, dtype=np.uint8)
    for (rows, cols, o_c, o_s, o_end) in ((2 * I, H, lay.w13, lay.s13, lay.w2),
                                          (H, I, lay.w2, lay.s2, lay.nbytes)):
        w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(sigma)
        c, g = encode_fp8(w)
        out[o_c:o_s] = c.reshape(-1)
        out[o_s:o_end] = _scale_field(g)
    return out


def _gauss_bf16_blob(rng: np.random.Generator, H: int, I: int, sigma: float) -> np.ndarray:
    lay = blob_layout(H, I, "bf16")
    w13 = f32_to_bf16_bits(rng.standard_normal((2 * I, H), dtype=np.float32) * np.float32(sigma))
    w2 = f32_to_bf16_bits(rng.standard_normal((H, I), dtype=np.float32) * np.float32(sigma))
    out = np.empty(lay.nbytes, dtype=np.uint8)
    out[lay.w13:lay.w2] = w13.reshape(-1).view(np.uint8)
    out[lay.w2:lay.nbytes] = w2.reshape(-1).view(np.uint8)
    return out


_MARGINAL_CACHE: dict = {}


def _marginal_tables(sigma: float):
    """Lookup tables whose outputs follow the marginal code / scale distributions
    of ``encode_mxfp4`` applied to N(0, sigma) (estimated once from a fixed sample).
    A uniform random byte indexes each table."""
    key = float(sigma)
    if key in _MARGINAL_CACHE:
        return _MARGINAL_CACHE[key]
    rng = _rng(12345, 99)
    sample = rng.standard_normal((4096, 1024), dtype=np.float32) * np.float32(sigma)
    packed, scales = encode_mxfp4(sample)
    codes = np.concatenate([packed & 15, packed >> 4]).reshape(-1)

    def lut_from(values: np.ndarray, nvals: int) -> np.ndarray:
        hist = np.bincount(values.reshape(-1).astype(np.int64), minlength=nvals).astype(np.float64)
        cdf = np.cumsum(hist) / hist.sum()
        u = (np.arange(256) + 0.5) / 256.0
        return np.searchsorted(cdf, u).astype(np.uint8)

    tabs = (lut_from(codes, 16), lut_from(scales, 256))
    _MARGINAL_CACHE[key] = tabs
    return tabs


def _marginal_mxfp4_blob(rng: np.random.Generator, H: int, I: int, sigma: float) -> np.ndarray:
    """Fast MXFP4 blob: independent codes and scales drawn from the marginals of
    quantised N(0, sigma). Used where a workload asks only for "MXFP4 weights"
    and is too large to quantise element by element."""
    lay = blob_layout(H, I, "mxfp4")
    code_lut, scale_lut = _marginal_tables(sigma)
    out = np.empty(lay.nbytes, dtype=np.uint8)
    nc13, ns13 = lay.s13 - lay.w13, lay.w2 - lay.s13
    nc2, ns2 = lay.s2 - lay.w2, lay.nbytes - lay.s2
    r = rng.integers(0, 256, size=(2, nc13 + nc2), dtype=np.uint8)
    codes = code_lut[r[0]] | (code_lut[r[1]] << 4)
    s = scale_lut[rng.integers(0, 256, size=ns13 + ns2, dtype=np.uint8)]
    out[lay.w13:lay.s13] = codes[:nc13]
    out[lay.w2:lay.s2] = codes[nc13:]
    out[lay.s13:lay.w2] = s[:ns13]
    out[lay.s2:lay.nbytes] = s[ns13:]
    return out


def _marginal_tables_fmt(fmt: str, sigma: float):
    """As _marginal_tables for NVFP4 (codes, block scales, matrix scale) and
    FP8 (codes, matrix scale)."""
    key = (fmt, float(sigma))
    if key in _MARGINAL_CACHE:
        return _MARGINAL_CACHE[key]
    rng = _rng(12345, 98)
    sample = rng.standard_normal((1024, 1024), dtype=np.float32) * np.float32(sigma)

    def lut_from(values: np.ndarray, nvals: int) -> np.ndarray:
        hist = np.bincount(values.reshape(-1).astype(np.int64), minlength=nvals).astype(np.float64)
        cdf = np.cumsum(hist) / hist.sum()
        u = (np.arange(256) + 0.5) / 256.0
        return np.searchsorted(cdf, u).astype(np.uint8)

    if fmt == "nvfp4":
        packed, sc, g = encode_nvfp4(sample)
        codes = np.concatenate([packed & 15, packed >> 4]).reshape(-1)
        tabs = (lut_from(codes, 16), lut_from(sc, 256), g)
    else:
        codes, g = encode_fp8(sample)
        tabs = (lut_from(codes, 256), None, g)
    _MARGINAL_CACHE[key] = tabs
    return tabs


def _marginal_nvfp4_blob(rng: np.random.Generator, H: int, I: int, sigma: float) -> np.ndarray:
    """Fast NVFP4 blob: independent codes and block scales from the marginals
    of quantised N(0, sigma), the sample's matrix scale."""
    lay = blob_layout(H, I, "nvfp4")
    code_lut, scale_lut, g = _marginal_tables_fmt("nvfp4", sigma)
    out = np.empty(lay.nbytes, dtype=np.uint8)
    for (rows, cols, o_c, o_s, o_end) in ((2 * I, H, lay.w13, lay.s13, lay.w2),
                                          (H, I, lay.w2, lay.s2, lay.nbytes)):
        r = rng.integers(0, 256, size=(2, rows * cols // 2), dtype=np.uint8)
        out[o_c:o_s] = code_lut[r[0]] | (code_lut[r[1]] << 4)
        ns = rows * cols // 16
        out[o_s:o_s + ns] = scale_lut[rng.integers(0, 256, size=ns, dtype=np.uint8)]
        out[o_s + ns:o_end] = _scale_field(g)
    return out


def _marginal_fp8_blob(rng: np.random.Generator, H: int, I: int, sigma: float) -> np.ndarray:
    lay = blob_layout(H, I, "fp8")
    code_lut, _, g = _marginal_tables_fmt("fp8", sigma)
    out = np.empty(lay.nbytes, dtype=np.uint8)
    for (rows, cols, o_c, o_s, o_end) in ((2 * I, H, lay.w13, lay.s13, lay.w2),
                                          (H, I, lay.w2, lay.s2, lay.nbytes)):
        out[o_c:o_s] = code_lut[rng.integers(0, 256, size=rows * cols, dtype=np.uint8)]
        out[o_s:o_end] = _scale_field(g)
    return out


def expert_blob(cfg: LayerConfig, layer: int, expert: int, shared: bool = False,
                H: int | None = None, I: int | None = None) -> np.ndarray:
    """One expert's blob (uint8 [nbytes]) in the storage layout of ``blob_layout``."""
    H = cfg.H if H is None else H
    I = cfg.I if I is None else I
    rng = _rng(cfg.wseed, _S_SHARED if shared else _S_W, layer, expert)
    if cfg.weights == "gauss_mxfp4":
        return _gauss_mxfp4_blob(rng, H, I, WEIGHT_SIGMA)
    if cfg.weights == "marginal_mxfp4":
        return _marginal_mxfp4_blob(rng, H, I, WEIGHT_SIGMA)
    if cfg.weights == "gauss_bf16":
        return _gauss_bf16_blob(rng, H, I, WEIGHT_SIGMA)
    if cfg.weights == "gauss_nvfp4":
        return _gauss_nvfp4_blob(rng, H, I, WEIGHT_SIGMA)
    if cfg.weights == "gauss_fp8":
        return _gauss_fp8_blob(rng, H, I, WEIGHT_SIGMA)
    if cfg.weights == "marginal_nvfp4":
        return _marginal_nvfp4_blob(rng, H, I, WEIGHT_SIGMA)
    if cfg.weights == "marginal_fp8":
        return _marginal_fp8_blob(rng, H, I, WEIGHT_SIGMA)
    raise ValueError(cfg.weights)


def expert_pool(cfg: LayerConfig, layer: int = 0, E: int | None = None, H: int | None = None,
                I: int | None = None) -> np.ndarray:
    """All routed experts of one layer, uint8 [E][nbytes], expert-major and contiguous."""
    E = cfg.E if E is None else E
    H = cfg.H if H is None else H
    I = cfg.I if I is None else I
    lay = blob_layout(H, I, cfg.fmt)
    pool = np.empty((E, lay.nbytes), dtype=np.uint8)

    def fill(e):
        pool[e] = expert_blob(cfg, layer, e, H=H, I=I)

    if E * lay.nbytes < (64 << 20):
        for e in range(E):
            fill(e)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range(E)))
    return pool


def shared_expert(cfg: LayerConfig, layer: int = 0, H: int | None = None,
                  I: int | None = None) -> np.ndarray:
    return expert_blob(cfg, layer, 0, shared=True, H=H, I=I)


# --------------------------------------------------------------------------
# Activations, gate weights, router logits
# --------------------------------------------------------------------------


def activations(cfg: LayerConfig, T: int, step: int = 0, H: int | None = None) -> np.ndarray:
    """x ~ N(0,1) rounded to bf16, uint16 [T][H]."""
    H = cfg.H if H is None else H
    rng = _rng(cfg.seed, _S_X, T, step)
    return f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))


def gate_weights(cfg: LayerConfig, layer: int = 0, E: int | None = None,
                 H: int | None = None) -> np.ndarray:
    """Router gate Wg ~ N(0, 0.02) rounded to bf16, uint16 [E][H]."""
    E = cfg.E if E is None else E
    H = cfg.H if H is None else H
    rng = _rng(cfg.seed, _S_GATE, layer)
    return f32_to_bf16_bits(rng.standard_normal((E, H), dtype=np.float32) * np.float32(GATE_SIGMA))


def zipf_permutation(cfg: LayerConfig, layer: int, phase: int, E: int | None = None) -> np.ndarray:
    E = cfg.E if E is None else E
    return _rng(cfg.seed, _S_PERM, layer, phase).permutation(E)


def router_logits(cfg: LayerConfig, T: int, step: int = 0, layer: int = 0,
                  E: int | None = None) -> np.ndarray:
    """fp32 router logits [T][E] drawn per the workload's popularity model.

    uniform     : iid U[0,1)               (flat popularity)
    gumbel_bias : b_e + Gumbel(0,1), b = 0.22 z, z ~ N(0,1), two dead experts at -30
    zipf        : log p_{pi(e)} + Gumbel(0,1), p_r ~ r^-1.1; pi re-drawn every 256 steps
    """
    E = cfg.E if E is None else E
    rng = _rng(cfg.seed, _S_LOGITS, T, step * 1000 + layer)
    if cfg.logits == "uniform":
        return rng.random((T, E), dtype=np.float32)
    if cfg.logits == "gumbel_bias":
        brng = _rng(cfg.seed, _S_BIAS, layer)
        b = BIAS_SCALE * brng.standard_normal(E)
        dead = brng.choice(E, size=2, replace=False)
        b[dead] = DEAD_EXPERT_BIAS
        return (b[None, :] + rng.gumbel(size=(T, E))).astype(np.float32)
    if cfg.logits == "zipf":
        pi = zipf_permutation(cfg, layer, step // ZIPF_PHASE_STEPS, E)
        ranks = np.arange(1, E + 1, dtype=np.float64)
        logp = -ZIPF_S * np.log(ranks)
        logp -= np.log(np.exp(logp).sum())
        return (logp[pi][None, :] + rng.gumbel(size=(T, E))).astype(np.float32)
    raise ValueError(f"config {cfg.name} draws logits from its gate")


def tie_logits(T: int, E: int, seed: int = 7) -> np.ndarray:
    """Logits on a coarse grid (multiples of 1/4 in [0, 2)) so that many tokens hold
    exact ties, including at the k / k+1 boundary."""
    rng = _rng(seed, 42)
    return (rng.integers(0, 8, size=(T, E)).astype(np.float32) / np.float32(4.0))


def pool_bytes(cfg: LayerConfig) -> int:
    """Bytes of all routed experts over all layers."""
    return cfg.layers * cfg.E * blob_layout(cfg.H, cfg.I, cfg.fmt).nbytes


def expected_unique_experts(E: int, k: int, T: int) -> float:
    """Distinct experts touched by T tokens with uniform top-k routing."""
    return E * (1.0 - (1.0 - k / E) ** T)


__all__ = [
    "LayerConfig", "CONFIGS", "BlobLayout", "blob_layout", "encode_mxfp4", "encode_nvfp4",
    "encode_fp8", "f32_to_bf16_bits",
    "expert_blob", "expert_pool", "shared_expert", "activations", "gate_weights",
    "router_logits", "zipf_permutation", "tie_logits", "pool_bytes", "expected_unique_experts",
]
