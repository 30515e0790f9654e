"""Host side of the bandwidth-adaptive placement, on the CPU: the host expert
kernel (moe_cpu_expert_ffn) against the oracle, and the split of a
permutation between the device and the host (moe_permute_split) against its
definition. Blobs reach the host kernel in the kernel layout, packed here by
an independent numpy re-derivation of the layout the header states."""
import numpy as np
import pytest

from mixture_experts_gate_amd import synth

from parity import assert_close, kernel_layout_mxfp4


@pytest.fixture(scope="module")
def lib():
    from mixture_experts_gate_amd import _lib
    return _lib


@pytest.mark.parametrize("H,I,E,n,weights", [(256, 256, 3, 5, "gauss_mxfp4"),
                                             (512, 384, 2, 1, "gauss_mxfp4"),
                                             (4096, 2048, 1, 2, "marginal_mxfp4")])
def test_cpu_expert_ffn_matches_oracle(lib, orc, H, I, E, n, weights):
    cfg = synth.LayerConfig("host_ffn", H, E, 2, I, "mxfp4", 0, "uniform", (n,), weights, seed=41)
    lay = synth.blob_layout(H, I, "mxfp4")
    pool = synth.expert_pool(cfg)
    packed = kernel_layout_mxfp4(pool, lay)
    x = synth.activations(cfg, 7, step=1)
    rng = np.random.default_rng(H)
    for e in range(E):
        rows = rng.choice(7, size=n, replace=True).astype(np.int32)
        xr = np.ascontiguousarray(x[rows])
        yr = np.zeros_like(xr)
        b = packed[e]
        base = b.ctypes.data
        lib.moe_cpu_expert_ffn(lib.MOE_W_MXFP4, base + lay.w13, base + lay.s13, base + lay.w2,
                               base + lay.s2, H, I, xr, yr, 2)
        ref = orc.ffn_rows(x, pool, lay, rows, np.full(n, e, dtype=np.int32))
        got = yr.view(np.uint16).astype(np.uint32) << 16
        assert_close(got.view(np.float32).astype(np.float64), ref, f"host expert {e} H={H} I={I}")


def test_cpu_expert_ffn_argument_errors(lib):
    x = np.zeros((1, 256), dtype=np.uint16)
    y = np.zeros_like(x)
    assert lib.load().moe_cpu_expert_ffn(lib.MOE_W_NVFP4, 1, 1, 1, 1, 256, 256,
                                         x.ctypes.data, 1, y.ctypes.data, 1) == lib.MOE_EUNSUPPORTED
    assert lib.load().moe_cpu_expert_ffn(lib.MOE_W_MXFP4, 1, 1, 1, 1, 250, 256,
                                         x.ctypes.data, 1, y.ctypes.data, 1) == lib.MOE_EINVAL
    assert lib.load().moe_cpu_expert_ffn(lib.MOE_W_MXFP4, None, 1, 1, 1, 256, 256,
                                         x.ctypes.data, 1, y.ctypes.data, 1) == lib.MOE_EINVAL


@pytest.mark.parametrize("T,E,k,seed", [(1, 8, 2, 0), (16, 32, 4, 1), (64, 128, 8, 2),
                                        (37, 256, 6, 3)])
def test_permute_split(lib, orc, T, E, k, seed):
    rng = np.random.default_rng(seed)
    lg = rng.random((T, E), dtype=np.float32)
    ids, _, _ = orc.topk(lg, k)
    off, sp, _ = orc.permute(ids, E)
    for frac in (0.0, 0.3, 1.0):
        mask = (rng.random(E) < frac).astype(np.uint8)
        d_off, d_sp, h_p = lib.moe_permute_split(off, sp, mask)
        cnt = np.diff(off)
        want_cnt = np.where(mask == 1, 0, cnt)
        assert np.array_equal(np.diff(d_off), want_cnt) and d_off[0] == 0
        assert np.array_equal(d_sp, np.concatenate(
            [sp[off[e]:off[e + 1]] for e in range(E) if not mask[e]] + [np.zeros(0, np.int32)]))
        assert np.array_equal(h_p, np.concatenate(
            [sp[off[e]:off[e + 1]] for e in range(E) if mask[e]] + [np.zeros(0, np.int32)]))
        assert sorted(np.concatenate([d_sp, h_p]).tolist()) == list(range(T * k))
