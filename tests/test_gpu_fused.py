"""The one-launch layer (moe_layer_fused: router from given logits, permutation,
expert FFN and combine in one persistent launch with a grid barrier) against
the CPU oracle and against the launch chain it replaces (moe_route +
moe_permute_ffn_combine), through the C ABI.

Routing ids, weights and the permutation must equal the chain's bit for bit
(the same device code computes them) and the oracle's (ids and permutation bit
for bit, weights within 1e-6); y and out must equal the chain's bit for bit
where both run the same gate/up tile shape (8 wavefronts per tile, which the
chain takes at these batch sizes) and lie within the stated tolerance of the
oracle's fp64 result everywhere. The barrier counters must count every call
and the wait-timeout flag never be set.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mixture_experts_gate_amd import synth  # noqa: E402

from parity import W_ATOL, assert_close, bf16_dev_to_f64, to_dev, to_dev_bf16  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _announce(msg):
    print(f"[gpu-fused] {msg}", flush=True)


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mixture_experts_gate_amd import _lib
    _lib.load()
    _lib.moe_set_option(_lib.MOE_OPT_FFN_PATH, 0)
    return _lib


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.build(force=False)
    return oracle


class Layer:
    def __init__(self, cfg):
        from mixture_experts_gate_amd.layer import DeviceExperts
        self.cfg = cfg
        self.lay = synth.blob_layout(cfg.H, cfg.I, cfg.fmt)
        self.pool = synth.expert_pool(cfg)
        self.dev = DeviceExperts(self.pool, self.lay, device=DEV)
        self.shared = synth.shared_expert(cfg) if cfg.n_shared else None
        self.dev_sh = DeviceExperts(self.shared, self.lay, device=DEV) if cfg.n_shared else None


_LAYERS = {}


def layer(name, H, E, k, I, shared, logits="uniform", weights="gauss_mxfp4", seed=71):
    key = (name, H, E, k, I, shared)
    if key not in _LAYERS:
        _announce(f"generating {name}: H={H} E={E} k={k} I={I} shared={shared}")
        cfg = synth.LayerConfig(name, H, E, k, I, "mxfp4", 1 if shared else 0, logits, (1,),
                                weights, seed=seed)
        _LAYERS[key] = Layer(cfg)
    return _LAYERS[key]


def new_sync():
    from mixture_experts_gate_amd import _lib
    return torch.zeros(_lib.LAYER_SYNC_BYTES // 8, dtype=torch.int64, device=DEV)


def check_sync(sync, calls):
    """After `calls` calls on a fresh sync buffer (256 workgroups, 16 groups of
    16): every group counted 16 arrivals per call, 16 groups completed per
    call, every release word holds the call count, no wait ran out."""
    w = sync.view(-1, 16)[:, 0].cpu().numpy()
    G = torch.cuda.get_device_properties(0).multi_processor_count
    assert w[33] == 0, "a barrier wait ran out"
    assert (w[:16] == calls * (G // 16)).all(), f"group arrivals {w[:16]}"
    assert w[16] == calls * 16, f"groups complete {w[16]}"
    assert (w[17:33] == calls).all(), f"release words {w[17:33]}"


def bufs(lib, c, T):
    n = T * c.k
    rows = n + (T if c.n_shared else 0)
    _, fb = lib.moe_workspace_size(T, c.k + 1 if c.n_shared else c.k, c.H, c.I, c.E)
    return dict(ids=torch.full((T, c.k), -5, dtype=torch.int32, device=DEV),
                w=torch.full((T, c.k), -5.0, dtype=torch.float32, device=DEV),
                off=torch.full((c.E + 1,), -5, dtype=torch.int32, device=DEV),
                sp=torch.full((n,), -5, dtype=torch.int32, device=DEV),
                pr=torch.full((n,), -5, dtype=torch.int32, device=DEV),
                y=torch.zeros((rows, c.H), dtype=torch.bfloat16, device=DEV),
                out=torch.zeros((T, c.H), dtype=torch.bfloat16, device=DEV),
                ws=torch.empty(fb, dtype=torch.uint8, device=DEV), fb=fb,
                sync=new_sync())


def fused(lib, L, T, x, lg, b, renorm=True, stream=None):
    c = L.cfg
    return lib.moe_layer_fused(x, lg, L.dev.table, L.dev_sh.table if L.dev_sh else None,
                               lib.MOE_W_MXFP4, T, c.k, c.H, c.I, c.E, renorm, b["ids"], b["w"],
                               b["off"], b["sp"], b["pr"], b["y"], b["out"], b["ws"], b["fb"],
                               b["sync"], stream, check=False)


def chain(lib, L, T, x, lg, b, renorm=True):
    c = L.cfg
    lib.moe_route(None, None, lg, None, T, c.H, c.E, c.k, renorm, b["ids"], b["w"])
    lib.moe_permute_ffn_combine(x, b["ids"], b["w"], L.dev.table,
                                L.dev_sh.table if L.dev_sh else None, lib.MOE_W_MXFP4, T, c.k,
                                c.H, c.I, c.E, b["off"], b["sp"], b["pr"], b["y"], b["out"],
                                b["ws"], b["fb"])


def check_vs_oracle(orc, L, T, x_np, lg_np, b, renorm=True):
    c = L.cfg
    ref = orc.moe_layer(x_np, L.lay, L.pool, c.k, logits=lg_np, shared_blob=L.shared,
                        renormalize=renorm)
    n = T * c.k
    assert np.array_equal(b["ids"].cpu().numpy(), ref["ids"]), "routing ids differ from the oracle"
    assert np.abs(b["w"].cpu().numpy().astype(np.float64) - ref["w"]).max() <= W_ATOL
    assert np.array_equal(b["off"].cpu().numpy(), ref["offsets"]), "offsets differ"
    assert np.array_equal(b["sp"].cpu().numpy(), ref["sorted_pair"]), "sorted_pair differs"
    assert np.array_equal(b["pr"].cpu().numpy(), ref["pair_row"]), "pair_row differs"
    assert_close(bf16_dev_to_f64(b["y"][:n]), ref["y"], f"y T={T}")
    assert_close(bf16_dev_to_f64(b["out"]), ref["out_f64"], f"out T={T}")


# (name, H, E, k, I, shared, T): the decode-shaped layer at one token, the
# large sparse layer at one and two tokens (six routed + the shared expert),
# and smaller shapes that take the other compiled tile shapes
_CASES = [
    ("decode", 2048, 128, 8, 768, False, 1),
    ("large_sparse", 4096, 256, 6, 2048, True, 1),
    ("large_sparse", 4096, 256, 6, 2048, True, 2),
    ("small", 1024, 64, 4, 512, False, 1),
    ("small", 1024, 64, 4, 512, False, 3),
    ("small", 1024, 64, 4, 512, True, 3),
    ("mid", 2048, 96, 3, 512, True, 2),
    ("wide", 4096, 200, 2, 768, False, 7),
    # 16 to 31 activation rows: two 16-row groups in the down part
    ("decode", 2048, 128, 8, 768, False, 2),
    ("decode", 2048, 128, 8, 768, False, 3),
    ("large_sparse", 4096, 256, 6, 2048, True, 3),
    ("large_sparse", 4096, 256, 6, 2048, True, 4),
    ("small", 1024, 64, 4, 512, True, 6),
    # the permutation's unrolled forms (up to 8, 16 and 31 routed pairs) at
    # their edges: 8 pairs + a shared row, 9, 17, 20 + 2 shared rows, 31
    ("small", 1024, 64, 8, 512, True, 1),
    ("small", 1024, 64, 3, 512, False, 3),
    ("mid", 2048, 96, 17, 512, False, 1),
    ("mid", 2048, 96, 10, 512, True, 2),
    ("small", 1024, 64, 31, 512, False, 1),
]


@pytest.mark.parametrize("name,H,E,k,I,shared,T", _CASES,
                         ids=[f"{c[0]}-H{c[1]}-E{c[2]}-k{c[3]}-I{c[4]}{'-sh' if c[5] else ''}-T{c[6]}"
                              for c in _CASES])
def test_fused_layer_vs_chain_and_oracle(lib, orc, name, H, E, k, I, shared, T):
    weights = "marginal_mxfp4" if name == "large_sparse" else "gauss_mxfp4"
    L = layer(name, H, E, k, I, shared, weights=weights)
    c = L.cfg
    for step in range(3):
        _announce(f"fused layer {name} H={H} E={E} k={k} I={I} shared={shared} T={T} step {step}")
        x_np = synth.activations(c, T, step=step)
        lg_np = synth.router_logits(c, T, step=step)
        x, lg = to_dev_bf16(x_np), to_dev(lg_np)
        a = bufs(lib, c, T)
        rc = fused(lib, L, T, x, lg, a)
        assert rc == 0, f"moe_layer_fused returned {rc}"
        torch.cuda.synchronize()
        check_sync(a["sync"], 1)
        b = bufs(lib, c, T)
        chain(lib, L, T, x, lg, b)
        torch.cuda.synchronize()
        for key in ("ids", "w", "off", "sp", "pr"):
            assert torch.equal(a[key], b[key]), f"{key} differs from the launch chain"
        rows = T * k + (T if shared else 0)
        if H // 128 in (16, 32) and rows <= 15:
            # the chain's gate/up tiles also split K over 8 wavefronts here,
            # and its down projection + combine is the same launch code
            for key in ("y", "out"):
                assert torch.equal(a[key], b[key]), f"{key} differs from the launch chain"
        else:
            # 8 slabs: the chain splits K over 4 wavefronts; from 16 rows its
            # down projection is the tiled weight-streaming launch (other fp32
            # orders)
            assert_close(bf16_dev_to_f64(a["out"]), bf16_dev_to_f64(b["out"]), "out vs chain")
        check_vs_oracle(orc, L, T, x_np, lg_np, a)


def test_fused_layer_no_renormalize(lib, orc):
    L = layer("decode", 2048, 128, 8, 768, False)
    c = L.cfg
    x_np = synth.activations(c, 1, step=5)
    lg_np = synth.router_logits(c, 1, step=5)
    a = bufs(lib, c, 1)
    assert fused(lib, L, 1, to_dev_bf16(x_np), to_dev(lg_np), a, renorm=False) == 0
    torch.cuda.synchronize()
    check_vs_oracle(orc, L, 1, x_np, lg_np, a, renorm=False)


def test_fused_layer_reuses_sync_and_workspace(lib, orc):
    """Consecutive calls on one sync buffer and workspace, alternating batch
    sizes and layers on one stream: each call's results as when run alone."""
    L4 = layer("large_sparse", 4096, 256, 6, 2048, True, weights="marginal_mxfp4")
    c = L4.cfg
    a = bufs(lib, c, 2)
    sync = a["sync"]
    outs = []
    for i, T in enumerate((2, 1, 2, 1, 1, 2)):
        x_np = synth.activations(c, T, step=10 + i)
        lg_np = synth.router_logits(c, T, step=10 + i)
        x, lg = to_dev_bf16(x_np), to_dev(lg_np)
        b = bufs(lib, c, T)
        b["ws"], b["fb"], b["sync"] = a["ws"], a["fb"], sync
        assert fused(lib, L4, T, x, lg, b) == 0
        outs.append((T, x, lg, b))
    torch.cuda.synchronize()
    check_sync(sync, 6)
    for T, x, lg, b in outs:
        r = bufs(lib, c, T)
        chain(lib, L4, T, x, lg, r)
        torch.cuda.synchronize()
        assert torch.equal(b["out"], r["out"]) and torch.equal(b["ids"], r["ids"])


def test_fused_layer_graph_replays(lib):
    """The launch captured in a HIP graph and replayed with new inputs copied
    into its buffers between replays (eager work and synchronisations in
    between): every replay equals the eager call on the same inputs, and the
    barrier counters are zero after each."""
    L = layer("decode", 2048, 128, 8, 768, False)
    c = L.cfg
    T = 1
    x = torch.empty((T, c.H), dtype=torch.bfloat16, device=DEV)
    lg = torch.empty((T, c.E), dtype=torch.float32, device=DEV)
    g_b = bufs(lib, c, T)
    s = torch.cuda.Stream()
    x.copy_(to_dev_bf16(synth.activations(c, T, step=0)))
    lg.copy_(to_dev(synth.router_logits(c, T, step=0)))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        assert fused(lib, L, T, x, lg, g_b, stream=s) == 0     # warm-up outside capture
        s.synchronize()
        with torch.cuda.graph(graph, stream=s):
            for _ in range(3):
                fused(lib, L, T, x, lg, g_b, stream=s)
    torch.cuda.synchronize()
    for r in range(5):
        _announce(f"graph replay {r}")
        xs = to_dev_bf16(synth.activations(c, T, step=20 + r))
        ls = to_dev(synth.router_logits(c, T, step=20 + r))
        x.copy_(xs)
        lg.copy_(ls)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        check_sync(g_b["sync"], 1 + 3 * (r + 1))
        e_b = bufs(lib, c, T)
        assert fused(lib, L, T, xs, ls, e_b) == 0
        torch.cuda.synchronize()
        for key in ("ids", "w", "off", "sp", "pr", "y", "out"):
            assert torch.equal(g_b[key], e_b[key]), f"replay {r}: {key} differs"


def test_fused_layer_declines_outside_its_sizes(lib):
    """Batches outside the one-launch sizes return MOE_EUNSUPPORTED and leave
    every output untouched."""
    L = layer("decode", 2048, 128, 8, 768, False)
    c = L.cfg
    T = 4                                   # 32 rows: more than the down part's two row groups
    b = bufs(lib, c, T)
    x = to_dev_bf16(synth.activations(c, T))
    lg = to_dev(synth.router_logits(c, T))
    assert fused(lib, L, T, x, lg, b) == lib.MOE_EUNSUPPORTED
    torch.cuda.synchronize()
    assert (b["ids"] == -5).all() and (b["off"] == -5).all() and not b["out"].float().any()


def test_layer_forward_takes_the_fused_launch(lib, orc):
    """MoeLayer.forward with given logits at one token runs the one-launch
    layer (one kernel launch) and matches the oracle."""
    from mixture_experts_gate_amd.layer import MoeLayer
    L = layer("large_sparse", 4096, 256, 6, 2048, True, weights="marginal_mxfp4")
    c = L.cfg
    M = MoeLayer(c.H, c.E, c.k, c.I, c.fmt, 2, shared=True, device=DEV)
    x_np = synth.activations(c, 1, step=3)
    lg_np = synth.router_logits(c, 1, step=3)
    torch.cuda.synchronize()
    lib.moe_set_option(lib.MOE_OPT_TIMING, 1)
    out = M.forward(1, to_dev_bf16(x_np), L.dev.table, logits=to_dev(lg_np),
                    shared_table=L.dev_sh.table)
    torch.cuda.synchronize()
    launched = lib.timing_report()
    lib.moe_set_option(lib.MOE_OPT_TIMING, 0)
    assert list(launched) == ["layer_fused"], f"launches: {launched}"
    ref = orc.moe_layer(x_np, L.lay, L.pool, c.k, logits=lg_np, shared_blob=L.shared)
    assert np.array_equal(M.topk_ids[:1].cpu().numpy(), ref["ids"])
    assert_close(bf16_dev_to_f64(out), ref["out_f64"], "forward out T=1")


@pytest.mark.parametrize("name,H,E,k,I,shared,T", [
    ("decode", 2048, 128, 8, 768, False, 1),
    ("large_sparse", 4096, 256, 6, 2048, True, 2),
])
def test_fused_layer_tied_logits(lib, orc, name, H, E, k, I, shared, T):
    """Logits with many exact ties (a few distinct values, signed zeros), so
    that the choice at the k boundary is decided by the lower expert index:
    ids and the permutation bit for bit against the oracle, out within the
    tolerance."""
    weights = "marginal_mxfp4" if name == "large_sparse" else "gauss_mxfp4"
    L = layer(name, H, E, k, I, shared, weights=weights)
    c = L.cfg
    rng = np.random.default_rng(99)
    lg_np = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 0.5, 1.0], np.float32), size=(T, E))
    x_np = synth.activations(c, T, step=7)
    a = bufs(lib, c, T)
    assert fused(lib, L, T, to_dev_bf16(x_np), to_dev(lg_np), a) == 0
    torch.cuda.synchronize()
    check_vs_oracle(orc, L, T, x_np, lg_np, a)


def test_fused_layer_deterministic(lib):
    """The same call twice on fresh buffers: every output bit for bit."""
    L = layer("large_sparse", 4096, 256, 6, 2048, True, weights="marginal_mxfp4")
    c = L.cfg
    x = to_dev_bf16(synth.activations(c, 2, step=8))
    lg = to_dev(synth.router_logits(c, 2, step=8))
    runs = []
    for _ in range(2):
        b = bufs(lib, c, 2)
        assert fused(lib, L, 2, x, lg, b) == 0
        runs.append(b)
    torch.cuda.synchronize()
    for key in ("ids", "w", "off", "sp", "pr", "y", "out"):
        assert torch.equal(runs[0][key], runs[1][key]), f"{key} differs between runs"
