"""The expert FFN entry point without a caller workspace (moe_expert_ffn_noalloc)
against moe_expert_ffn with a workspace, through the C ABI: the same kernels
run, so the expert outputs must agree bit for bit. Two calls in a row, the
second with a smaller batch (the tiled kernels, then the weight-streaming
ones), each checked; a request whose workspace exceeds the library's array is
refused before any device work."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mixture_experts_gate_amd import synth  # noqa: E402

from parity import to_dev, to_dev_bf16  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def env():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_gate_amd import _lib
    from mixture_experts_gate_amd.layer import DeviceExperts
    _lib.load()
    _lib.moe_set_option(_lib.MOE_OPT_FFN_PATH, 0)
    c = synth.CONFIGS[2]
    lay = synth.blob_layout(c.H, c.I, c.fmt)
    pool = synth.expert_pool(c)
    return dict(lib=_lib, cfg=c, lay=lay, dev=DeviceExperts(pool, lay, device=DEV))


def _routed(env, T, step):
    from mixture_experts_gate_amd.layer import MoeLayer
    c = env["cfg"]
    L = MoeLayer(c.H, c.E, c.k, c.I, c.fmt, T, device=DEV)
    x = to_dev_bf16(synth.activations(c, T, step=step))
    L.route_permute(T, logits=to_dev(synth.router_logits(c, T, step=step)))
    return L, x


def test_noalloc_matches_workspace_call_twice(env):
    lib, c = env["lib"], env["cfg"]
    tab = env["dev"].table
    for T in (2048, 64):          # tiled kernels first, then the smaller decode batch
        print(f"[no-alloc] T={T}", flush=True)
        L, x = _routed(env, T, step=T)
        _, need = lib.moe_workspace_size(T, c.k, c.H, c.I, c.E)
        assert need <= lib.FFN_NOALLOC_MAX_WS
        n = T * c.k
        y_ws = torch.full((n, c.H), float("nan"), dtype=torch.bfloat16, device=DEV)
        y_na = torch.full((n, c.H), float("nan"), dtype=torch.bfloat16, device=DEV)
        lib.moe_expert_ffn(x, L.sorted_pair, L.offsets, tab, L.fmt, T, c.k, c.H, c.I, c.E, y_ws,
                           False, L.ws_ffn, L.ws_ffn_bytes)
        lib.moe_expert_ffn_noalloc(x, L.sorted_pair, L.offsets, tab, L.fmt, T, c.k, c.H, c.I,
                                   c.E, y_na, False)
        torch.cuda.synchronize()
        assert not torch.isnan(y_ws.float()).any()
        assert torch.equal(y_ws, y_na), f"T={T}: outputs differ"


def test_noalloc_refuses_oversized_request(env):
    lib, c = env["lib"], env["cfg"]
    T = 8192
    _, need = lib.moe_workspace_size(T, c.k, c.H, c.I, c.E)
    assert need > lib.FFN_NOALLOC_MAX_WS
    y = torch.empty((1, c.H), dtype=torch.bfloat16, device=DEV)
    dummy = torch.zeros(T * c.k, dtype=torch.int32, device=DEV)
    off = torch.zeros(c.E + 1, dtype=torch.int32, device=DEV)
    x = torch.zeros((T, c.H), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(lib.MoeError) as ei:
        lib.moe_expert_ffn_noalloc(x, dummy, off, env["dev"].table, lib.MOE_W_MXFP4, T, c.k, c.H,
                                   c.I, c.E, y, False)
    assert ei.value.code == lib.MOE_ENOMEM
