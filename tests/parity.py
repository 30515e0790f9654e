"""Shared helpers for the GPU parity tests: device upload of seeded inputs and
the error measures the tolerances are stated in."""
from __future__ import annotations

import numpy as np

# Tolerance for floating-point outputs: the layer's output (bf16, fp32
# accumulation) must satisfy max|got - ref| / max|ref| <= 2e-2 against the
# oracle's exact (fp64) result.
MAX_REL = 2e-2
# Tighter bound derived from the arithmetic: bf16 rounding of the SwiGLU
# activation, of each expert output and of the final sum each contribute at
# most 2^-9 relative error per element, so the L2-relative error of a correct
# kernel stays well under 1e-2 (a dropped K block or expert term does not).
L2_REL = 1e-2
# Routing weights: fp32 exp on the GPU vs double in the oracle.
W_ATOL = 1e-6


def max_rel(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def l2_rel(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


def assert_close(got, ref, what: str):
    mr, lr = max_rel(got, ref), l2_rel(got, ref)
    print(f"  {what}: max-rel {mr:.3e}  l2-rel {lr:.3e}", flush=True)
    assert mr <= MAX_REL, f"{what}: max-rel {mr:.3e} > {MAX_REL}"
    assert lr <= L2_REL, f"{what}: l2-rel {lr:.3e} > {L2_REL}"


def to_dev_bf16(bits: np.ndarray, dev="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def to_dev(a: np.ndarray, dev="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_dev_to_f64(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def kernel_layout_mxfp4(blobs, lay):
    """Interchange MXFP4 blobs [n][nbytes] -> the kernel layout the library's
    header states (16-row x 128-column blocks, lane l = row l % 16, columns
    32 (l / 16) .. + 31), re-derived here with numpy for the host-side tests."""
    def tiled(codes, scales, R, K):
        nslab = K // 128
        c = codes.reshape(R // 16, 16, nslab, 4, 16)           # rb, row, s, cb, byte
        oc = c.transpose(0, 2, 3, 1, 4).reshape(-1)            # rb, s, lane=(cb,row), byte
        sc = scales.reshape(R // 16, 16, nslab, 4).transpose(0, 2, 3, 1).reshape(-1)
        return oc, sc

    blobs = np.atleast_2d(blobs)
    out = np.empty_like(blobs)
    H, I = lay.H, lay.I
    for e in range(blobs.shape[0]):
        b = blobs[e]
        c13, s13 = tiled(b[lay.w13:lay.s13], b[lay.s13:lay.w2], 2 * I, H)
        c2, s2 = tiled(b[lay.w2:lay.s2], b[lay.s2:lay.nbytes], H, I)
        out[e, lay.w13:lay.s13], out[e, lay.s13:lay.w2] = c13, s13
        out[e, lay.w2:lay.s2], out[e, lay.s2:lay.nbytes] = c2, s2
    return out
