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
