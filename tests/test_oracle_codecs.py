"""Pins for the oracle's number codecs (MXFP4 elements and scales, bf16 rounding).

The expected values come from the published element grid of OCP Microscaling
v1.0 (E2M1: 0, 0.5, 1, 1.5, 2, 3, 4, 6 with a sign bit; E8M0: power-of-two
scale with bias 127, 0xFF = NaN), from torch's fp32->bf16 rounding (a library
routine), and from hand-worked bf16 bit patterns.
"""
import math

import numpy as np
import pytest
import torch

from mixture_experts_gate_amd import synth

# OCP MX v1.0 E2M1 magnitudes indexed by the 3 low bits of the code
E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_all_codes(orc):
    for code in range(16):
        mag = E2M1_SPEC[code & 7]
        want = -mag if code & 8 else mag
        got = orc.e2m1(code)
        assert got == want, (code, got, want)
        if code == 8:
            assert math.copysign(1.0, got) == -1.0  # negative zero keeps its sign


def test_e8m0_all_scales(orc):
    assert orc.e8m0(127) == 1.0
    assert math.isnan(orc.e8m0(255))
    prev = orc.e8m0(0)
    assert prev > 0
    for s in range(1, 255):
        v = orc.e8m0(s)
        assert v == 2.0 * prev, s          # each step doubles
        m, _ = math.frexp(v)
        assert m == 0.5                    # exact power of two
        prev = v
    assert orc.e8m0(254) == 2.0 ** 127


def _lut_decode(codes, scales, R, K):
    """Independent decode: table lookup of the spec grid, layout as stored
    (row-major, even element in the low nibble, one scale per 32 along K)."""
    lut = np.array(E2M1_SPEC + [-v for v in E2M1_SPEC], dtype=np.float64)
    c = np.empty((R, K), dtype=np.int64)
    c[:, 0::2] = codes.reshape(R, K // 2) & 15
    c[:, 1::2] = codes.reshape(R, K // 2) >> 4
    sc = np.repeat(scales.reshape(R, K // 32).astype(np.int64), 32, axis=1)
    return lut[c] * np.exp2(sc - 127.0)


def test_mxfp4_decode_matrix_matches_lut(orc):
    rng = np.random.default_rng(3)
    R, K = 7, 96
    codes = rng.integers(0, 256, size=(R, K // 2), dtype=np.uint8)
    scales = rng.integers(90, 160, size=(R, K // 32), dtype=np.uint8)
    got = orc.mxfp4_decode(codes, scales, R, K)
    want = _lut_decode(codes, scales, R, K)
    assert np.array_equal(got, want)


def test_mxfp4_decode_every_code_every_scale(orc):
    # one row per scale 0..254, each row walks all 16 codes twice
    R, K = 255, 32
    codes = np.tile(np.array([(2 * i) & 15 | (((2 * i + 1) & 15) << 4) for i in range(16)],
                             dtype=np.uint8), (R, 1))
    scales = np.arange(255, dtype=np.uint8).reshape(R, 1)
    got = orc.mxfp4_decode(codes, scales, R, K)
    want = _lut_decode(codes, scales, R, K)
    assert np.array_equal(got, want)


def test_encoder_roundtrip_error_bound(orc):
    """The generator's quantiser and the oracle's decoder agree on layout: the
    decoded value lies within half a grid step (times the block scale) of the
    input, and exactly on it where the input is on the grid."""
    rng = np.random.default_rng(11)
    w = rng.standard_normal((16, 256)).astype(np.float32) * np.float32(0.02)
    codes, scales = synth.encode_mxfp4(w)
    dec = orc.mxfp4_decode(codes, scales, 16, 256)
    sc = np.repeat(np.exp2(scales.astype(np.float64) - 127.0), 32, axis=1)
    q = np.abs(w.astype(np.float64)) / sc
    step = np.where(q < 2, 0.5, np.where(q < 4, 1.0, 2.0))
    err = np.abs(dec - w) / sc
    # saturation only happens above 6 (a block's max maps into [4, 8))
    assert (err[q <= 6] <= (step / 2)[q <= 6] + 1e-12).all()
    assert (np.abs(dec[q > 6]) / sc[q > 6] == 6.0).all()
    # on-grid inputs decode exactly
    grid = np.array(E2M1_SPEC, dtype=np.float32)
    wg = (grid[rng.integers(0, 8, size=(4, 64))] * np.float32(2.0 ** -6)).astype(np.float32)
    wg[:, ::32] = 6.0 * 2.0 ** -6          # pin each block's max so the scale is 2^-6
    c2, s2 = synth.encode_mxfp4(wg)
    assert (s2 == 127 - 6).all()
    assert np.array_equal(orc.mxfp4_decode(c2, s2, 4, 64), wg.astype(np.float64))


@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
    (1.0 + 2.0 ** -8, 0x3F80),           # tie -> even (mantissa 0)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),       # tie -> even (mantissa 2)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),  # just above the tie rounds up
    (3.0e38 * 1.2, 0x7F80),              # beyond the overflow midpoint -> inf
    (2.0 ** -133, 0x0001),               # smallest subnormal
    (2.0 ** -134, 0x0000),               # half of it: tie -> even (zero)
    (1.5 * 2.0 ** -134, 0x0001),
])
def test_bf16_known_patterns(orc, value, bits):
    assert orc.f64_to_bf16(value) == bits


def test_bf16_matches_torch_on_fp32_values(orc):
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(4000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-38).astype(np.float32),
                        rng.integers(0, 2 ** 32, size=3000, dtype=np.uint64).astype(np.uint32)
                        .view(np.float32)])
    v = v[np.isfinite(v)]
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f64_to_bf16(float(a)) for a in v], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_bf16_to_f64_exact(orc):
    for bits in (0x3F80, 0xC000, 0x0001, 0x7F7F, 0x4049):
        t = torch.from_numpy(np.array([bits], dtype=np.uint16).view(np.int16))
        want = float(t.view(torch.bfloat16).float())
        assert orc.bf16_to_f64(bits) == want


# ------------------------------------------------------------ E4M3, NVFP4, FP8 --

def _torch_e4m3(codes):
    """torch's float8_e4m3fn -> float64 (library routine)."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_all_codes_match_torch(orc):
    want = _torch_e4m3(np.arange(256, dtype=np.uint8))
    for c in range(256):
        got = orc.e4m3(c)
        if c & 0x7F == 0x7F:
            assert math.isnan(got) and math.isnan(want[c]), c
        else:
            assert got == want[c], (c, got, want[c])
            assert math.copysign(1.0, got) == math.copysign(1.0, want[c]), c


@pytest.mark.parametrize("code,value", [
    (0x38, 1.0), (0x3C, 1.5), (0x40, 2.0), (0x7E, 448.0), (0x01, 2.0 ** -9),
    (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0xB8, -1.0), (0x30, 0.5),
])
def test_e4m3_closed_forms(orc, code, value):
    """(1 + m/8) 2^(e-7) for normal codes, m/8 2^-6 for subnormal ones."""
    assert orc.e4m3(code) == value


def test_nvfp4_worked_example(orc):
    """Two 16-element blocks of one row, hand-computed: block 0 has scale 0x38
    (1.0), block 1 has 0x44 (3.0); matrix scale 0.5."""
    codes = np.zeros(16, np.uint8)
    codes[0] = 0x1 | (0x2 << 4)          # elements 0, 1: 0.5, 1.0
    codes[7] = 0xF | (0x7 << 4)          # elements 14, 15: -6, 6
    codes[8] = 0x3 | (0xB << 4)          # elements 16, 17: 1.5, -1.5
    codes[15] = 0x5 | (0x0 << 4)         # elements 30, 31: 3, 0
    scales = np.array([0x38, 0x44], np.uint8)
    got = orc.nvfp4_decode(codes, scales, 0.5, 1, 32)[0]
    want = np.zeros(32)
    want[0], want[1], want[14], want[15] = 0.25, 0.5, -3.0, 3.0
    want[16], want[17], want[30] = 2.25, -2.25, 4.5
    assert np.array_equal(got, want)


def test_nvfp4_block_structure(orc):
    """Changing the scale byte of block b of row r changes exactly elements
    16b..16b+15 of row r, by the ratio of the two scales; g scales everything."""
    rng = np.random.default_rng(5)
    R, K = 3, 64
    codes = rng.integers(0, 256, size=(R, K // 2), dtype=np.uint8)
    scales = rng.integers(0x20, 0x50, size=(R, K // 16), dtype=np.uint8)
    base = orc.nvfp4_decode(codes, scales, 1.0, R, K)
    assert np.array_equal(orc.nvfp4_decode(codes, scales, 0.25, R, K), base * 0.25)
    for r, b in ((0, 0), (1, 3), (2, 2)):
        s2 = scales.copy()
        s2[r, b] = 0x38 if scales[r, b] != 0x38 else 0x40
        d = orc.nvfp4_decode(codes, s2, 1.0, R, K)
        changed = np.zeros((R, K), bool)
        changed[r, 16 * b:16 * b + 16] = True
        assert np.array_equal(d[~changed], base[~changed])
        ratio = orc.e4m3(s2[r, b]) / orc.e4m3(scales[r, b])
        assert np.array_equal(d[changed], base[changed] * ratio)


def test_nvfp4_encoder_roundtrip_error_bound(orc):
    """The generator's quantiser and the oracle's decoder agree on layout: every
    decoded value lies within one E2M1 grid unit (at the block's decoded scale)
    of the input."""
    rng = np.random.default_rng(13)
    w = rng.standard_normal((16, 256)).astype(np.float32) * np.float32(0.02)
    codes, scales, g = synth.encode_nvfp4(w)
    dec = orc.nvfp4_decode(codes, scales, g, 16, 256)
    unit = np.repeat(_torch_e4m3(scales), 16, axis=1) * float(g)
    assert (np.abs(dec - w) <= unit + 1e-12).all()
    # and much closer on average than a wrong block mapping would be
    assert np.abs(dec - w).mean() < 0.2 * np.abs(w).mean()


def test_fp8_decode_matches_torch(orc):
    rng = np.random.default_rng(17)
    R, K = 5, 64
    codes = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38          # no NaN codes in weights
    got = orc.fp8_decode(codes, 0.375, R, K)
    assert np.array_equal(got, _torch_e4m3(codes) * 0.375)


def test_fp8_encoder_roundtrip_error_bound(orc):
    rng = np.random.default_rng(19)
    w = rng.standard_normal((8, 128)).astype(np.float32) * np.float32(0.02)
    codes, g = synth.encode_fp8(w)
    dec = orc.fp8_decode(codes, g, 8, 128)
    # E4M3 keeps 4 significant bits: relative error <= 2^-4 above the subnormals
    big = np.abs(w) > float(g) * 2.0 ** -6
    assert (np.abs(dec - w)[big] <= 2.0 ** -4 * np.abs(w)[big] + 1e-12).all()
    assert (np.abs(dec - w)[~big] <= float(g) * 2.0 ** -10 + 1e-12).all()
