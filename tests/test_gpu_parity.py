"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Routing ids, permutation offsets / order / inverse are compared bit for bit;
routing weights within 1e-6; floating-point outputs by max-relative error
(<= 2e-2, the stated tolerance) and L2-relative error (<= 1e-2, from the bf16
roundings). Large workloads are checked in full for routing and permutation
and on sampled tokens for the FFN and combine (the layer is token-independent
once routing is fixed, which the oracle tests pin).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mixture_experts_gate_amd import synth  # noqa: E402

from parity import W_ATOL, assert_close, bf16_dev_to_f64, to_dev, to_dev_bf16  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _announce(msg):
    print(f"[gpu-parity] {msg}", flush=True)


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


class Workload:
    """Weights of one layer, generated once and resident on the device."""

    def __init__(self, cfg, E=None):
        from mixture_experts_gate_amd.layer import DeviceExperts
        self.cfg = cfg
        self.E = cfg.E if E is None else E
        self.lay = synth.blob_layout(cfg.H, cfg.I, cfg.fmt)
        self.pool = synth.expert_pool(cfg, E=self.E)
        self.dev = DeviceExperts(self.pool, self.lay, device=DEV)
        self.shared = synth.shared_expert(cfg) if cfg.n_shared else None
        self.dev_shared = DeviceExperts(self.shared, self.lay, device=DEV) if cfg.n_shared else None


_WL = {}


def workload(c, E=None):
    key = (c, E)
    if key not in _WL:
        _announce(f"generating weights for config {c} (E={E})")
        _WL[key] = Workload(synth.CONFIGS[c], E)
    return _WL[key]


def run_layer(w: Workload, T, x, logits=None, wg=None, y_fp32=False, renormalize=True,
              fused=True, fuse_shared=True, fuse_combine=True):
    from mixture_experts_gate_amd.layer import MoeLayer
    cfg = w.cfg
    L = MoeLayer(cfg.H, w.E, cfg.k, cfg.I, cfg.fmt, T, shared=bool(cfg.n_shared), y_fp32=y_fp32,
                 device=DEV)
    xd = to_dev_bf16(x)
    out = L.forward(T, xd, w.dev.table,
                    logits=None if logits is None else to_dev(logits),
                    wg=None if wg is None else to_dev_bf16(wg),
                    shared_table=w.dev_shared.table if w.dev_shared else None,
                    renormalize=renormalize, write_logits=True, fused_routing=fused,
                    fuse_shared=fuse_shared, fuse_combine=fuse_combine)
    torch.cuda.synchronize()
    return L, out


def oracle_tokens(orc, w: Workload, x, ids, wts, toks):
    """Oracle FFN + combine for the listed tokens (its own routing ids / weights)."""
    k = w.cfg.k
    toks = np.asarray(toks, dtype=np.int32)
    rt = np.repeat(toks, k)
    re_ = ids[toks].reshape(-1)
    y = orc.ffn_rows(x, w.pool, w.lay, rt, re_)
    ysh = None
    if w.shared is not None:
        ysh = orc.ffn_rows(x, w.shared[None], w.lay, toks, np.zeros(len(toks), np.int32))
    out, _ = orc.combine(y, wts[toks], ysh)
    return y, out


def check_routing(L, T, ref_ids, ref_w, logits_ref=None):
    ids = L.topk_ids[:T].cpu().numpy()
    assert np.array_equal(ids, ref_ids), "routing ids differ"
    w = L.topk_w[:T].cpu().numpy()
    assert np.abs(w.astype(np.float64) - ref_w).max() <= W_ATOL
    if logits_ref is not None:
        assert np.array_equal(L.logits[:T].cpu().numpy(), logits_ref), "logits differ"


def check_permutation(L, T, E, ref_off, ref_sp, ref_pr):
    n = T * L.k
    assert np.array_equal(L.offsets.cpu().numpy(), ref_off), "offsets differ"
    assert np.array_equal(L.sorted_pair[:n].cpu().numpy(), ref_sp), "sorted_pair differs"
    assert np.array_equal(L.pair_row[:n].cpu().numpy(), ref_pr), "pair_row differs"


# ------------------------------------------------------------------ router --

@pytest.mark.parametrize("fused", [True, False])
def test_route_gate_tiny_bitwise(lib, orc, fused):
    _announce(f"route: tiny config, bf16 gate on GPU (fused={fused})")
    w = workload(1)
    cfg = w.cfg
    x = synth.activations(cfg, 16)
    wg = synth.gate_weights(cfg)
    L, _ = run_layer(w, 16, x, wg=wg, fused=fused)
    lg = orc.gate_logits_f32(x, wg)
    ids, wts, _ = orc.topk(lg, cfg.k)
    check_routing(L, 16, ids, wts, logits_ref=lg)


@pytest.mark.parametrize("T,H,E", [(3, 2048, 128), (37, 4096, 256), (5, 64, 1000)])
def test_route_gate_shapes_bitwise(lib, orc, T, H, E):
    _announce(f"route: gate GEMV T={T} H={H} E={E}")
    rng = np.random.default_rng(T)
    x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wg = synth.f32_to_bf16_bits((rng.standard_normal((E, H)) * 0.02).astype(np.float32))
    k = 6
    ids_d = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w_d = torch.empty((T, k), dtype=torch.float32, device=DEV)
    lg_d = torch.empty((T, E), dtype=torch.float32, device=DEV)
    lib.moe_route(to_dev_bf16(x), to_dev_bf16(wg), None, lg_d, T, H, E, k, True, ids_d, w_d)
    torch.cuda.synchronize()
    lg = orc.gate_logits_f32(x, wg)
    assert np.array_equal(lg_d.cpu().numpy(), lg)
    ids, wts, _ = orc.topk(lg, k)
    assert np.array_equal(ids_d.cpu().numpy(), ids)
    assert np.abs(w_d.cpu().numpy().astype(np.float64) - wts).max() <= W_ATOL


ROUTE_CASES = [
    ("cfg2-T64", lambda: synth.router_logits(synth.CONFIGS[2], 64), 8, True),
    ("cfg3-T8192", lambda: synth.router_logits(synth.CONFIGS[3], 8192), 8, True),
    ("cfg4-T4096", lambda: synth.router_logits(synth.CONFIGS[4], 4096), 6, True),
    ("ties", lambda: synth.tie_logits(500, 16), 5, True),
    ("ties-k-boundary", lambda: synth.tie_logits(300, 64), 8, True),
    ("no-renorm", lambda: synth.router_logits(synth.CONFIGS[4], 100), 6, False),
    ("k=E", lambda: synth.router_logits(synth.CONFIGS[2], 20, E=8), 8, True),
    ("k=1", lambda: synth.router_logits(synth.CONFIGS[2], 50), 1, True),
    ("E=1000", lambda: np.random.default_rng(4).random((33, 1000), dtype=np.float32), 7, True),
    ("signed-zero", lambda: np.tile(np.array([[-0.0, 0.0, -1.0, 0.0, 0.5]], np.float32), (4, 1)), 3,
     True),
]


@pytest.mark.parametrize("name,make,k,renorm", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_logits_bitwise(lib, orc, name, make, k, renorm):
    _announce(f"route: {name}")
    lg = make()
    T, E = lg.shape
    ids_d = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w_d = torch.empty((T, k), dtype=torch.float32, device=DEV)
    lib.moe_route(None, None, to_dev(lg), None, T, 0, E, k, renorm, ids_d, w_d)
    torch.cuda.synchronize()
    ids, wts, _ = orc.topk(lg, k, renormalize=renorm)
    assert np.array_equal(ids_d.cpu().numpy(), ids)
    assert np.abs(w_d.cpu().numpy().astype(np.float64) - wts).max() <= W_ATOL


# ------------------------------------------------------------- permutation --

def _perm_case(T, E, k, kind, seed=0):
    rng = np.random.default_rng(seed + T)
    if kind == "uniform":
        lg = rng.random((T, E), dtype=np.float32)
    elif kind == "skew":   # one expert takes every token's first slot, many experts empty
        lg = rng.random((T, E), dtype=np.float32)
        lg[:, 3] += 10.0
        lg[:, E // 2:] -= 10.0
    else:
        raise ValueError(kind)
    return lg


PERM_CASES = [(1, 128, 8, "uniform"), (8, 128, 8, "uniform"), (64, 128, 8, "uniform"),
              (16, 8, 2, "uniform"), (500, 256, 6, "skew"), (513, 512, 4, "uniform"),
              (4096, 256, 6, "uniform"), (8192, 128, 8, "uniform"), (6000, 64, 3, "skew"),
              (1, 1, 1, "uniform"), (3, 7, 7, "uniform"), (33, 128, 8, "uniform"),
              (48, 64, 4, "skew"), (64, 512, 6, "skew"), (100, 128, 8, "skew"),
              (256, 128, 8, "uniform"), (250, 64, 4, "skew"), (257, 128, 8, "uniform"),
              (2, 512, 6, "uniform"), (5, 512, 8, "skew"), (8, 33, 8, "uniform"),
              (4, 64, 16, "skew")]


@pytest.mark.parametrize("T,E,k,kind", PERM_CASES)
def test_permute_bitwise(lib, orc, T, E, k, kind):
    _announce(f"permute: T={T} E={E} k={k} {kind}")
    lg = _perm_case(T, E, k, kind)
    ids, _, _ = orc.topk(lg, k)
    off, sp, pr = orc.permute(ids, E)
    pb, _ = lib.moe_workspace_size(T, k, 64, 64, E)
    ws = torch.empty(max(pb, 256), dtype=torch.uint8, device=DEV)
    off_d = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    sp_d = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    pr_d = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    lib.moe_permute(to_dev(ids), T, k, E, off_d, sp_d, pr_d, ws, max(pb, 256))
    torch.cuda.synchronize()
    assert np.array_equal(off_d.cpu().numpy(), off)
    assert np.array_equal(sp_d.cpu().numpy(), sp)
    assert np.array_equal(pr_d.cpu().numpy(), pr)


@pytest.mark.parametrize("T,E,k,kind", [c for c in PERM_CASES if c[0] * c[2] <= 4096])
def test_route_permute_fused_bitwise(lib, orc, T, E, k, kind):
    _announce(f"route+permute fused: T={T} E={E} k={k} {kind}")
    lg = _perm_case(T, E, k, kind)
    ids, wts, _ = orc.topk(lg, k)
    off, sp, pr = orc.permute(ids, E)
    ids_d = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
    w_d = torch.empty((T, k), dtype=torch.float32, device=DEV)
    off_d = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    sp_d = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    pr_d = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    lib.moe_route_permute(None, None, to_dev(lg), None, T, 0, E, k, True, ids_d, w_d, off_d, sp_d,
                          pr_d, ws, 256)
    torch.cuda.synchronize()
    assert np.array_equal(ids_d.cpu().numpy(), ids)
    assert np.abs(w_d.cpu().numpy().astype(np.float64) - wts).max() <= W_ATOL
    assert np.array_equal(off_d.cpu().numpy(), off)
    assert np.array_equal(sp_d.cpu().numpy(), sp)
    assert np.array_equal(pr_d.cpu().numpy(), pr)


def test_route_permute_reuses_workspace(lib, orc):
    """Consecutive router + permutation calls on one workspace, with batch
    sizes that take the one-workgroup kernels and the separate router and
    permutation (one-workgroup and chunked), logits given and the gate
    computed: each call equals the oracle bit for bit, whatever the calls
    before it left in the workspace."""
    E, k, H = 256, 6, 512
    pb, _ = lib.moe_workspace_size(1000, k, H, 64, E)
    pb = max(pb, 256)
    ws = torch.zeros(pb, dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(17)
    wg = synth.f32_to_bf16_bits((rng.standard_normal((E, H)) * 0.02).astype(np.float32))
    for i, (T, gate) in enumerate([(64, False), (33, False), (600, False), (5, False), (9, False),
                                   (37, True), (64, False), (12, True), (20, True), (257, False),
                                   (1000, False), (64, False)]):
        _announce(f"route+permute, shared workspace: call {i}, T={T}, gate={gate}")
        x = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
        lg = orc.gate_logits_f32(x, wg) if gate else rng.random((T, E), dtype=np.float32)
        ids, wts, _ = orc.topk(lg, k)
        off, sp, pr = orc.permute(ids, E)
        ids_d = torch.full((T, k), -7, dtype=torch.int32, device=DEV)
        w_d = torch.empty((T, k), dtype=torch.float32, device=DEV)
        off_d = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
        sp_d = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
        pr_d = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
        if gate:
            lib.moe_route_permute(to_dev_bf16(x), to_dev_bf16(wg), None, None, T, H, E, k, True,
                                  ids_d, w_d, off_d, sp_d, pr_d, ws, pb)
        else:
            lib.moe_route_permute(None, None, to_dev(lg), None, T, 0, E, k, True, ids_d, w_d,
                                  off_d, sp_d, pr_d, ws, pb)
        torch.cuda.synchronize()
        assert np.array_equal(ids_d.cpu().numpy(), ids)
        assert np.abs(w_d.cpu().numpy().astype(np.float64) - wts).max() <= W_ATOL
        assert np.array_equal(off_d.cpu().numpy(), off)
        assert np.array_equal(sp_d.cpu().numpy(), sp)
        assert np.array_equal(pr_d.cpu().numpy(), pr)


def test_permute_empty_batch(lib):
    off_d = torch.full((9,), -7, dtype=torch.int32, device=DEV)
    lib.moe_permute(None, 0, 2, 8, off_d, None, None, None, 0)
    torch.cuda.synchronize()
    assert (off_d.cpu().numpy() == 0).all()


# ------------------------------------------------------------- whole layer --

def _check_layer_full(orc, w, T, x, L, out, logits=None, wg=None):
    cfg = w.cfg
    ref = orc.moe_layer(x, w.lay, w.pool, cfg.k, logits=logits, wg=wg,
                        shared_blob=w.shared)
    check_routing(L, T, ref["ids"], ref["w"], logits_ref=ref["logits"])
    check_permutation(L, T, w.E, ref["offsets"], ref["sorted_pair"], ref["pair_row"])
    yg = L.y[:T * cfg.k].float().cpu().numpy()
    assert_close(yg, ref["y"], f"expert outputs y (T={T})")
    assert_close(bf16_dev_to_f64(out), ref["out_f64"], f"layer output (T={T})")
    return ref


def test_layer_tiny_bf16(lib, orc):
    _announce("layer: tiny bf16 config, T=16")
    w = workload(1)
    x = synth.activations(w.cfg, 16)
    wg = synth.gate_weights(w.cfg)
    L, out = run_layer(w, 16, x, wg=wg)
    _check_layer_full(orc, w, 16, x, L, out, wg=wg)


@pytest.mark.parametrize("T,fused", [(1, True), (8, True), (32, True), (64, True), (64, False)])
def test_layer_decode_cfg2(lib, orc, T, fused):
    _announce(f"layer: decode config 2, T={T} (fused routing={fused})")
    w = workload(2)
    x = synth.activations(w.cfg, T)
    lg = synth.router_logits(w.cfg, T)
    L, out = run_layer(w, T, x, logits=lg, fused=fused)
    _check_layer_full(orc, w, T, x, L, out, logits=lg)


def test_layer_decode_cfg2_fp32_y(lib, orc):
    _announce("layer: decode config 2, T=32, fp32 expert outputs")
    w = workload(2)
    x = synth.activations(w.cfg, 32, step=1)
    lg = synth.router_logits(w.cfg, 32, step=1)
    L, out = run_layer(w, 32, x, logits=lg, y_fp32=True)
    _check_layer_full(orc, w, 32, x, L, out, logits=lg)


def _check_layer_sampled(orc, w, T, x, lg, L, out, n_sample=24, seed=0):
    cfg = w.cfg
    ids, wts, _ = orc.topk(lg, cfg.k)
    off, sp, pr = orc.permute(ids, w.E)
    check_routing(L, T, ids, wts)
    check_permutation(L, T, w.E, off, sp, pr)
    rng = np.random.default_rng(seed)
    toks = np.sort(rng.choice(T, size=min(n_sample, T), replace=False))
    toks[-1] = T - 1    # always include the ragged tail's last token
    y_ref, out_ref = oracle_tokens(orc, w, x, ids, wts, toks)
    yg = L.y[:T * cfg.k].float().cpu().numpy().reshape(T, cfg.k, cfg.H)[toks].reshape(-1, cfg.H)
    assert_close(yg, y_ref, f"expert outputs y, {len(toks)} sampled tokens (T={T})")
    assert_close(bf16_dev_to_f64(out)[toks], out_ref, f"layer output, sampled (T={T})")


def test_layer_prefill_cfg3(lib, orc):
    _announce("layer: prefill config 3, T=8192")
    w = workload(3)
    T = 8192
    x = synth.activations(w.cfg, T)
    lg = synth.router_logits(w.cfg, T)
    L, out = run_layer(w, T, x, logits=lg)
    _check_layer_sampled(orc, w, T, x, lg, L, out)


@pytest.mark.parametrize("T", [1, 2, 64])
def test_layer_large_sparse_cfg4(lib, orc, T):
    """Config 4 (Zipf routing, shared expert) at decode sizes, every token
    against the oracle: at T=64 the hottest experts' rows span several 16-row
    blocks, and checking all tokens covers every row of every block."""
    _announce(f"layer: config 4 (shared expert, Zipf), T={T}, all tokens")
    w = workload(4)
    x = synth.activations(w.cfg, T)
    lg = synth.router_logits(w.cfg, T)
    L, out = run_layer(w, T, x, logits=lg)
    ids, _, _ = orc.topk(lg, w.cfg.k)
    if T == 64:
        assert np.bincount(ids.ravel(), minlength=w.E).max() > 16   # experts over one block
    _check_layer_sampled(orc, w, T, x, lg, L, out, n_sample=T)


def test_layer_cfg4_uniform_shared_blocks(lib, orc):
    """Config 4's shapes with uniform routing at T=40: no routed expert over 16
    rows, so the shared expert enters the routed launches as three 16-token
    blocks (the 8-wavefront gate/up and 64-row down kernels with the shared
    path), sampled tokens against the oracle."""
    _announce("layer: config 4 shapes, uniform routing, T=40 (shared expert in blocks)")
    w = workload(4)
    T = 40
    x = synth.activations(w.cfg, T, step=9)
    lg = np.random.default_rng(40).random((T, w.E), dtype=np.float32)
    L, out = run_layer(w, T, x, logits=lg)
    ids, _, _ = orc.topk(lg, w.cfg.k)
    assert np.bincount(ids.ravel(), minlength=w.E).max() <= 16
    _check_layer_sampled(orc, w, T, x, lg, L, out, n_sample=8)
    toks = np.array([0, 17, 39], dtype=np.int32)
    ysh_ref = orc.ffn_rows(x, w.shared[None], w.lay, toks, np.zeros(len(toks), np.int32))
    ysh = L.y[T * w.cfg.k + toks].float().cpu().numpy()
    assert_close(ysh, ysh_ref, "shared expert rows (three blocks)")


def _tile_rows(off, hot, n_rest, tile, rng):
    """Sorted rows to check on the tiled path: the first and last row of every
    `tile`-row tile of the `hot` experts with most rows, and the first and last
    row of `n_rest` other non-empty experts (their last, partial tiles)."""
    cnt = np.diff(off)
    order = np.argsort(-cnt, kind="stable")
    rows = set()
    for e in order[:hot]:
        for t0 in range(off[e], off[e + 1], tile):
            rows.update((t0, min(t0 + tile, off[e + 1]) - 1))
    rest = [e for e in order[hot:] if cnt[e] > 0]
    pick = rng.choice(len(rest), size=min(n_rest, len(rest)), replace=False)
    for i in pick:
        e = rest[i]
        rows.update((off[e], off[e + 1] - 1))
    coldest = [e for e in order[::-1] if cnt[e] > 0][0]
    rows.update((off[coldest], off[coldest + 1] - 1))
    return np.array(sorted(rows), dtype=np.int64)


def _check_rows(orc, w, x, L, rows, off, sp):
    """Expert outputs y of the given sorted rows against the oracle, row by row."""
    k = w.cfg.k
    e_of = np.searchsorted(off, rows, side="right") - 1
    pairs = sp[rows]
    y_ref = orc.ffn_rows(x, w.pool, w.lay, (pairs // k).astype(np.int32),
                         e_of.astype(np.int32))
    yg = L.y[torch.from_numpy(pairs).to(DEV)].float().cpu().numpy()
    assert_close(yg, y_ref, f"expert outputs y of {len(rows)} rows chosen by tile")


def test_layer_large_sparse_cfg4_T4096(lib, orc):
    """Config 4 at T=4096 (tiled kernels, Zipf routing: the hottest expert holds
    about 3000 rows, the coldest a handful): routing and permutation in full;
    expert outputs of the first and last row of every 64-row tile of the three
    hottest experts and of the first and last rows of 40 other experts (their
    partial last tiles) and the coldest; the layer output on sampled tokens."""
    _announce("layer: config 4, T=4096, rows chosen by tile")
    w = workload(4)
    T = 4096
    x = synth.activations(w.cfg, T)
    lg = synth.router_logits(w.cfg, T)
    L, out = run_layer(w, T, x, logits=lg)
    _check_layer_sampled(orc, w, T, x, lg, L, out, n_sample=8)
    ids, _, _ = orc.topk(lg, w.cfg.k)
    off, sp, _ = orc.permute(ids, w.E)
    rows = _tile_rows(off, 3, 40, 64, np.random.default_rng(4096))
    _check_rows(orc, w, x, L, rows, off, sp)


@pytest.mark.parametrize("path", [1, 2])
def test_ffn_paths_agree_with_oracle(lib, orc, path):
    """Both FFN implementations on one ragged workload: an expert with more
    than 64 tokens (several weight passes in the decode kernels), empty
    experts, a partial last tile."""
    _announce(f"ffn: forced path {path}, skewed T=300 on 16 experts")
    w = workload(2, E=16)
    T = 300
    x = synth.activations(w.cfg, T, step=5)
    lg = _perm_case(T, 16, 8, "skew")
    lib.moe_set_option(lib.MOE_OPT_FFN_PATH, path)
    try:
        L, out = run_layer(w, T, x, logits=lg)
    except lib.MoeError as e:
        if e.code == lib.MOE_EUNSUPPORTED:
            pytest.skip("this FFN path is not available for the shape")
        raise
    finally:
        lib.moe_set_option(lib.MOE_OPT_FFN_PATH, 0)
    _check_layer_sampled(orc, w, T, x, lg, L, out, n_sample=20)


@pytest.mark.parametrize("path", [1, 2])
def test_ffn_paths_odd_tile_counts(lib, orc, path):
    """H = 768, I = 384: three 256-row down tiles (the tiled path's two-tile
    workgroups fall back to one), 6- and 3-slab contractions, skewed routing."""
    _announce(f"ffn: forced path {path}, H=768 I=384 E=16 k=4 T=400")
    cfg = synth.LayerConfig("odd_tiles", 768, 16, 4, 384, "mxfp4", 0, "uniform", (400,),
                            "gauss_mxfp4", seed=7)
    w = Workload(cfg)
    T = 400
    x = synth.activations(cfg, T, step=1)
    lg = _perm_case(T, 16, 4, "skew")
    lib.moe_set_option(lib.MOE_OPT_FFN_PATH, path)
    try:
        L, out = run_layer(w, T, x, logits=lg)
    finally:
        lib.moe_set_option(lib.MOE_OPT_FFN_PATH, 0)
    _check_layer_sampled(orc, w, T, x, lg, L, out, n_sample=16)


def test_shared_expert_call_is_plain_swiglu(lib, orc):
    _announce("ffn: E=1, k=1 identity call (shared-expert form)")
    w = workload(4)
    T = 40
    x = synth.activations(w.cfg, T, step=2)
    from mixture_experts_gate_amd.layer import MoeLayer
    M = MoeLayer(w.cfg.H, w.cfg.E, w.cfg.k, w.cfg.I, w.cfg.fmt, T, shared=True, device=DEV)
    M.prepare_shared(T)
    M.shared_ffn(T, to_dev_bf16(x), w.dev_shared.table)
    torch.cuda.synchronize()
    ref = orc.ffn_rows(x, w.shared[None], w.lay, np.arange(T, dtype=np.int32),
                       np.zeros(T, np.int32))
    assert_close(M.y_sh[:T].float().cpu().numpy(), ref, "shared expert y")


@pytest.mark.parametrize("c,T", [(1, 16), (2, 1), (2, 64), (3, 8192), (4, 64), (4, 4096)])
def test_layer_deterministic(lib, c, T):
    """The same layer call twice gives bit-identical routing, permutation,
    expert outputs and layer output (no order-deciding atomics anywhere):
    the weight-streaming kernels, the tiled kernels (configs 3 and 4 at large
    T) and the shared expert in both forms."""
    _announce(f"determinism: config {c} T={T} twice")
    w = workload(c)
    x = synth.activations(w.cfg, T, step=3)
    if c == 1:
        kw = dict(wg=synth.gate_weights(w.cfg))
    else:
        kw = dict(logits=synth.router_logits(w.cfg, T, step=3))
    L1, o1 = run_layer(w, T, x, **kw)
    a = (o1.clone(), L1.y.clone(), L1.sorted_pair.clone(), L1.pair_row.clone(),
         L1.offsets.clone(), L1.topk_w.clone())
    L2, o2 = run_layer(w, T, x, **kw)
    b = (o2, L2.y, L2.sorted_pair, L2.pair_row, L2.offsets, L2.topk_w)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("T,fuse_shared", [(64, True), (64, False), (1, True), (2, True)])
def test_layer_graph_replays(lib, T, fuse_shared):
    """Graph replays of the layer (config 4, its shared expert in the routed
    launches or as its own call on a side stream; at T=1 and 2 the down
    projection and the combine in one launch) repeat the eager result
    exactly, with eager calls on the same buffers between the replays."""
    _announce(f"graph replays of config 4 T={T} against the eager result (fused={fuse_shared})")
    from mixture_experts_gate_amd.layer import MoeLayer
    w = workload(4)
    x = to_dev_bf16(synth.activations(w.cfg, T, step=6))
    lg = to_dev(synth.router_logits(w.cfg, T, step=6))
    L = MoeLayer(w.cfg.H, w.E, w.cfg.k, w.cfg.I, w.cfg.fmt, T, shared=True, device=DEV)
    L.prepare_shared(T)
    ref = L.forward(T, x, w.dev.table, logits=lg, shared_table=w.dev_shared.table,
                    fuse_shared=fuse_shared).clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        L.forward(T, x, w.dev.table, logits=lg, shared_table=w.dev_shared.table,
                  fuse_shared=fuse_shared)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = L.forward(T, x, w.dev.table, logits=lg, shared_table=w.dev_shared.table,
                        fuse_shared=fuse_shared)
    for r in range(4):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {r} differs from the eager result"
        # eager work on the same buffers between replays
        L.forward(T, x, w.dev.table, logits=lg, shared_table=w.dev_shared.table,
                  fuse_shared=fuse_shared)
        torch.cuda.synchronize()
        assert torch.equal(L.out[:T], ref)


def test_pack_mxfp4_layout(lib):
    """The kernel layout as the header states it, built independently in numpy
    from random interchange bytes."""
    _announce("pack: interchange -> kernel MXFP4 layout")
    H, I, n = 256, 384, 3
    lay = synth.blob_layout(H, I, "mxfp4")
    rng = np.random.default_rng(21)
    src = rng.integers(0, 256, size=(n, lay.nbytes), dtype=np.uint8)

    def tiled(codes, scales, R, K):
        nslab = K // 128
        c = codes.reshape(R // 16, 16, nslab, 4, 16)          # rb, row, s, cb, byte
        oc = c.transpose(0, 2, 3, 1, 4).reshape(-1)              # rb, s, lane=(cb,row), byte
        sc = scales.reshape(R // 16, 16, nslab, 4).transpose(0, 2, 3, 1).reshape(-1)
        return oc, sc

    want = np.empty_like(src)
    for e in range(n):
        b = src[e]
        c13, s13 = tiled(b[lay.w13:lay.s13], b[lay.s13:lay.w2], 2 * I, H)
        c2, s2 = tiled(b[lay.w2:lay.s2], b[lay.s2:lay.nbytes], H, I)
        want[e, lay.w13:lay.s13], want[e, lay.s13:lay.w2] = c13, s13
        want[e, lay.w2:lay.s2], want[e, lay.s2:lay.nbytes] = c2, s2
    d_src = to_dev(src)
    d_dst = torch.zeros_like(d_src)
    lib.moe_pack_mxfp4(d_src, d_dst, n, lay.nbytes, lay.nbytes, H, I, lay)
    torch.cuda.synchronize()
    assert np.array_equal(d_dst.cpu().numpy(), want)


# ------------------------------------------------------- NVFP4 and FP8 weights --

_FMT_CASES = [
    # (fmt, H, I, E, k, T, logits kind)
    # the decode layer's shapes (16- and 6-slab contractions, 64-row down tiles
    # at T=64, 32-row tiles and 8-wavefront gate/up at T=1)
    ("nvfp4", 2048, 768, 128, 8, 64, "uniform"),
    ("nvfp4", 2048, 768, 128, 8, 1, "uniform"),
    ("fp8", 2048, 768, 128, 8, 64, "uniform"),
    ("fp8", 2048, 768, 128, 8, 1, "uniform"),
    ("nvfp4", 1024, 512, 16, 4, 1, "uniform"),
    ("nvfp4", 1024, 512, 16, 4, 64, "uniform"),
    ("nvfp4", 768, 384, 16, 4, 200, "skew"),
    ("fp8", 1024, 512, 16, 4, 1, "uniform"),
    ("fp8", 1024, 512, 16, 4, 64, "uniform"),
    ("fp8", 768, 384, 16, 4, 200, "skew"),
]


@pytest.mark.parametrize("fmt,H,I,E,k,T,kind", _FMT_CASES,
                         ids=[f"{c[0]}-H{c[1]}-I{c[2]}-T{c[5]}-{c[6]}" for c in _FMT_CASES])
def test_layer_nvfp4_fp8_weights(lib, orc, fmt, H, I, E, k, T, kind):
    """Layers whose experts are stored in NVFP4 or FP8 (weight-streaming
    kernels), against the oracle's exact decode: small and large batches,
    skewed routing with several token passes per expert, 6/3- and 8/4-slab
    contractions."""
    _announce(f"layer: {fmt} weights H={H} I={I} E={E} k={k} T={T} ({kind})")
    cfg = synth.LayerConfig(f"{fmt}_test", H, E, k, I, fmt, 0, "uniform", (T,), "gauss_" + fmt,
                            seed=23)
    w = Workload(cfg)
    x = synth.activations(cfg, T, step=2)
    lg = synth.router_logits(cfg, T, step=2) if kind == "uniform" else _perm_case(T, E, k, kind)
    L, out = run_layer(w, T, x, logits=lg)
    _check_layer_full(orc, w, T, x, L, out, logits=lg)


_FC_CASES = [
    # (fmt, H, I, E, k, shared, T, logits kind)
    ("mxfp4", 2048, 768, 128, 8, False, 1, "uniform"),   # the decode layer at one token
    ("mxfp4", 1024, 2048, 32, 6, True, 2, "uniform"),    # 16-slab contraction, 14 rows
    ("mxfp4", 2048, 768, 128, 4, False, 3, "skew"),      # one expert in every token's first slot
    ("mxfp4", 512, 256, 16, 1, False, 1, "uniform"),     # one active expert, seven idle wavefronts
    ("mxfp4", 512, 256, 16, 2, True, 5, "skew"),         # 15 rows, the shared expert's 5
    ("nvfp4", 1024, 512, 16, 4, True, 3, "uniform"),
    ("fp8", 1024, 1024, 16, 4, False, 3, "skew"),        # 8 slabs
    ("fp8", 2048, 768, 128, 8, False, 1, "uniform"),
    ("mxfp4", 2048, 768, 128, 8, False, 2, "uniform"),   # 16 rows: the two calls
    ("mxfp4", 512, 256, 16, 1, False, 17, "uniform"),    # more than 16 tokens: the two calls
]


@pytest.mark.parametrize("fmt,H,I,E,k,shared,T,kind", _FC_CASES,
                         ids=[f"{c[0]}-H{c[1]}-I{c[2]}-E{c[3]}-k{c[4]}{'-sh' if c[5] else ''}"
                              f"-T{c[6]}-{c[7]}" for c in _FC_CASES])
def test_ffn_combine(lib, orc, fmt, H, I, E, k, shared, T, kind):
    """moe_expert_ffn_combine (the layer's default FFN + combine): y rows, the
    shared expert's rows and the layer output against the oracle; the output
    against the same layer through moe_expert_ffn + moe_combine (within the
    tolerance; equal bit for bit where the batch takes the two calls); a
    repeat call equal bit for bit."""
    _announce(f"ffn+combine: {fmt} H={H} I={I} E={E} k={k} shared={shared} T={T} {kind}")
    cfg = synth.LayerConfig(f"fc_{fmt}", H, E, k, I, fmt, 1 if shared else 0, "uniform", (T,),
                            "gauss_" + fmt, seed=37)
    w = Workload(cfg)
    x = synth.activations(cfg, T, step=6)
    lg = synth.router_logits(cfg, T, step=6) if kind == "uniform" else _perm_case(T, E, k, kind)
    L, out = run_layer(w, T, x, logits=lg)
    _check_layer_full(orc, w, T, x, L, out, logits=lg)
    out_a = out.clone()
    if shared:
        ysh_ref = orc.ffn_rows(x, w.shared[None], w.lay, np.arange(T, dtype=np.int32),
                               np.zeros(T, np.int32))
        assert_close(L.y[T * k:T * k + T].float().cpu().numpy(), ysh_ref, "shared expert rows")
    L2, out2 = run_layer(w, T, x, logits=lg, fuse_combine=False)
    o1, o2 = bf16_dev_to_f64(out_a), bf16_dev_to_f64(out2)
    two_calls = T > 16 or T * k + (T if shared else 0) > 15
    if two_calls:
        assert np.array_equal(o1, o2), "the two-call fallback differs from the two calls"
    else:
        assert_close(o1, o2, "fused against the two calls")
    L3, out3 = run_layer(w, T, x, logits=lg)
    assert torch.equal(out3, out_a), "repeat call differs"
    assert torch.equal(L3.y[:T * k], L.y[:T * k])


_SHARED_CASES = [("mxfp4", 1, "uniform", False), ("mxfp4", 7, "uniform", False),
                 ("mxfp4", 17, "skew", False), ("mxfp4", 40, "uniform", True),
                 ("bf16", 9, "uniform", False), ("nvfp4", 20, "uniform", False),
                 ("fp8", 33, "skew", False)]


@pytest.mark.parametrize("fmt,T,kind,y_fp32", _SHARED_CASES,
                         ids=[f"{c[0]}-T{c[1]}-{c[2]}{'-f32' if c[3] else ''}"
                              for c in _SHARED_CASES])
def test_ffn_shared_in_routed_launch(lib, orc, fmt, T, kind, y_fp32):
    """The shared expert as one more expert of the routed launches
    (moe_expert_ffn_shared): every routed row and every shared row against the
    oracle, the layer output too, and the same layer with the shared expert as
    its own call. T > 16 takes the shared expert through several token passes."""
    _announce(f"ffn+shared one launch: {fmt} T={T} {kind} y_fp32={y_fp32}")
    H, I, E, k = 512, 256, 16, 4
    cfg = synth.LayerConfig(f"shared_{fmt}", H, E, k, I, fmt, 1, "uniform", (T,), "gauss_" + fmt,
                            seed=31)
    w = Workload(cfg)
    x = synth.activations(cfg, T, step=4)
    lg = synth.router_logits(cfg, T, step=4) if kind == "uniform" else _perm_case(T, E, k, kind)
    L, out = run_layer(w, T, x, logits=lg, y_fp32=y_fp32)
    ref = _check_layer_full(orc, w, T, x, L, out, logits=lg)
    ysh_ref = orc.ffn_rows(x, w.shared[None], w.lay, np.arange(T, dtype=np.int32),
                           np.zeros(T, np.int32))
    ysh = L.y[T * k:T * k + T].float().cpu().numpy()
    assert_close(ysh, ysh_ref, f"shared expert rows (T={T})")
    L2, out2 = run_layer(w, T, x, logits=lg, y_fp32=y_fp32, fuse_shared=False)
    assert_close(bf16_dev_to_f64(out2), ref["out_f64"], f"layer output, separate shared call")
    assert_close(L2.y_sh[:T].float().cpu().numpy(), ysh_ref, "shared rows, separate call")


@pytest.mark.parametrize("T,k,shared", [(200, 1, False), (200, 1, True), (45, 2, True)])
def test_decode_multipass_one_hot_expert(lib, orc, T, k, shared):
    """Weight-streaming kernels with every token's first choice on one expert
    (up to 13 blocks of 16 rows): the expert's blocks, each its own entry of
    the active set, must cover every row exactly once, and every block must
    load its own token operand."""
    _announce(f"decode, one hot expert over many blocks: T={T} k={k} shared={shared}")
    H, I, E = 256, 128, 16
    cfg = synth.LayerConfig("one_hot", H, E, k, I, "mxfp4", int(shared), "uniform", (T,),
                            "gauss_mxfp4", seed=33)
    w = Workload(cfg)
    x = synth.activations(cfg, T, step=7)
    lg = np.random.default_rng(T).random((T, E), dtype=np.float32)
    lg[:, 5] += 10.0
    lib.moe_set_option(lib.MOE_OPT_FFN_PATH, 1)
    try:
        L, out = run_layer(w, T, x, logits=lg)
    finally:
        lib.moe_set_option(lib.MOE_OPT_FFN_PATH, 0)
    _check_layer_full(orc, w, T, x, L, out, logits=lg)


@pytest.mark.parametrize("E,k,T,kind,shared", [
    (512, 8, 64, "uniform", False),   # every group of 64 experts in the active set
    (500, 6, 40, "skew", True),       # a partial last group; one hot expert over 3 blocks
    (65, 4, 33, "uniform", False),    # the second group holds one expert
    (1, 1, 40, "uniform", True),      # a single expert: 3 blocks, plus the shared expert's 3
])
def test_decode_block_set_shapes(lib, orc, E, k, T, kind, shared):
    """Weight-streaming kernels (forced) on expert counts that exercise the
    block set's groups of 64 experts: all eight groups, a partial last
    group, a single expert split into several blocks; every token against
    the oracle."""
    _announce(f"decode block set: E={E} k={k} T={T} {kind} shared={shared}")
    H, I = 256, 128
    cfg = synth.LayerConfig("blocks", H, E, k, I, "mxfp4", int(shared), "uniform", (T,),
                            "gauss_mxfp4", seed=41)
    w = Workload(cfg)
    x = synth.activations(cfg, T, step=3)
    lg = synth.router_logits(cfg, T, step=3) if kind == "uniform" or E < 8 else \
        _perm_case(T, E, k, kind)
    lib.moe_set_option(lib.MOE_OPT_FFN_PATH, 1)
    try:
        L, out = run_layer(w, T, x, logits=lg)
    finally:
        lib.moe_set_option(lib.MOE_OPT_FFN_PATH, 0)
    _check_layer_full(orc, w, T, x, L, out, logits=lg)
    if shared:
        ysh_ref = orc.ffn_rows(x, w.shared[None], w.lay, np.arange(T, dtype=np.int32),
                               np.zeros(T, np.int32))
        assert_close(L.y[T * k:T * k + T].float().cpu().numpy(), ysh_ref, "shared expert rows")


@pytest.mark.parametrize("T,kind", [(24, "uniform"), (300, "skew")])
def test_ffn_shared_in_tiled_launch(lib, orc, T, kind):
    """The tiled kernels (forced) with the shared expert as expert E of the
    token-tile map: every routed and every shared row against the oracle, the
    layer output too, and the same layer with the shared expert as its own
    call on a side stream."""
    _announce(f"ffn+shared one tiled launch: T={T} ({kind})")
    H, I, E, k = 512, 256, 16, 4
    cfg = synth.LayerConfig("shared_tiled", H, E, k, I, "mxfp4", 1, "uniform", (T,),
                            "gauss_mxfp4", seed=32)
    w = Workload(cfg)
    x = synth.activations(cfg, T, step=1)
    lg = synth.router_logits(cfg, T, step=1) if kind == "uniform" else _perm_case(T, E, k, kind)
    lib.moe_set_option(lib.MOE_OPT_FFN_PATH, 2)
    try:
        L, out = run_layer(w, T, x, logits=lg)
        L2, out2 = run_layer(w, T, x, logits=lg, fuse_shared=False)
    finally:
        lib.moe_set_option(lib.MOE_OPT_FFN_PATH, 0)
    ref = _check_layer_full(orc, w, T, x, L, out, logits=lg)
    ysh_ref = orc.ffn_rows(x, w.shared[None], w.lay, np.arange(T, dtype=np.int32),
                           np.zeros(T, np.int32))
    assert_close(L.y[T * k:T * k + T].float().cpu().numpy(), ysh_ref, f"shared rows (T={T})")
    assert_close(bf16_dev_to_f64(out2), ref["out_f64"], "layer output, separate shared call")


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_pack_nvfp4_fp8_layout(lib, fmt):
    """The kernel layouts of NVFP4 and FP8 as the header states them, built
    independently in numpy from random interchange bytes."""
    _announce(f"pack: interchange -> kernel {fmt} layout")
    H, I, n = 256, 384, 3
    lay = synth.blob_layout(H, I, fmt)
    rng = np.random.default_rng(22)
    src = rng.integers(0, 256, size=(n, lay.nbytes), dtype=np.uint8)

    def nv(codes, scales, R, K):
        nslab = K // 128
        c = codes.reshape(R // 16, 16, nslab, 4, 16)           # rb, row, s, cb, byte
        oc = c.transpose(0, 2, 3, 1, 4).reshape(-1)
        sc = scales.reshape(R // 16, 16, nslab, 4, 2).transpose(0, 2, 3, 1, 4).reshape(-1)
        return oc, sc

    def f8(codes, R, K):
        nslab = K // 128
        c = codes.reshape(R // 16, 16, nslab, 4, 32)           # rb, row, s, cb, byte
        return c.transpose(0, 2, 3, 1, 4).reshape(-1)

    want = src.copy()       # the fp32 scale fields stay where they are
    for e in range(n):
        b = src[e]
        for (R, K, oc, os_) in ((2 * I, H, lay.w13, lay.s13), (H, I, lay.w2, lay.s2)):
            if fmt == "nvfp4":
                c, sc = nv(b[oc:os_], b[os_:os_ + R * K // 16], R, K)
                want[e, oc:os_], want[e, os_:os_ + R * K // 16] = c, sc
            else:
                want[e, oc:os_] = f8(b[oc:os_], R, K)
    d_src = to_dev(src)
    d_dst = torch.zeros_like(d_src)
    lib.moe_pack_weights(lib.MOE_W_NVFP4 if fmt == "nvfp4" else lib.MOE_W_FP8, d_src, d_dst, n,
                         lay.nbytes, lay.nbytes, H, I, lay)
    torch.cuda.synchronize()
    assert np.array_equal(d_dst.cpu().numpy(), want)


@pytest.mark.parametrize("H,I,E,k,T,kind,path", [
    (768, 384, 16, 4, 400, "skew", 2),       # forced onto the tiled kernels; 3 down tiles
    (1024, 512, 16, 4, 2048, "uniform", 0),  # chosen by size
    (2048, 768, 128, 8, 8192, "prefill", 0), # the prefill workload's shapes: 16/6 slabs
])
def test_fp8_weights_tiled_path(lib, orc, H, I, E, k, T, kind, path):
    """FP8 experts on the tiled (matrix-core) kernels: E4M3 weights with unit
    block scales and the matrix scale on the sums, against the oracle on
    sampled tokens (the last one included)."""
    _announce(f"layer: fp8 weights, tiled path, H={H} I={I} E={E} k={k} T={T} ({kind})")
    cfg = synth.LayerConfig("fp8_tiled", H, E, k, I, "fp8", 0, "uniform", (T,), "gauss_fp8",
                            seed=29)
    w = Workload(cfg)
    x = synth.activations(cfg, T, step=3)
    if kind == "uniform":
        lg = synth.router_logits(cfg, T, step=3)
    elif kind == "prefill":     # the prefill workload's routing (biased Gumbel, dead experts)
        lg = synth.router_logits(synth.CONFIGS[3], T)
    else:
        lg = _perm_case(T, E, k, kind)
    lib.moe_set_option(lib.MOE_OPT_FFN_PATH, path)
    try:
        L, out = run_layer(w, T, x, logits=lg)
    finally:
        lib.moe_set_option(lib.MOE_OPT_FFN_PATH, 0)
    _check_layer_sampled(orc, w, T, x, lg, L, out, n_sample=12)
    if kind == "prefill":
        ids, _, _ = orc.topk(lg, k)
        off, sp, _ = orc.permute(ids, E)
        rows = _tile_rows(off, 2, 24, 64, np.random.default_rng(T))
        _check_rows(orc, w, x, L, rows, off, sp)


# (H, I, E, k, shared, T, ids kind)
_PFC_CASES = [
    (2048, 768, 128, 8, False, 64, "uniform"),   # the decode layer at its headline batch
    (2048, 768, 128, 8, False, 9, "uniform"),    # 72 pairs
    (1024, 512, 128, 8, False, 2, "uniform"),    # 16 pairs: the smallest in-launch batch
    (1024, 512, 65, 4, False, 33, "hot"),        # a 33-row expert (three blocks); E % 64 != 0
    (1024, 512, 256, 6, True, 40, "zipf"),       # shared expert: 240 pairs + 40 shared rows
    (512, 256, 16, 8, False, 64, "hot"),         # 512 pairs, a 64-row expert (four blocks)
    (512, 256, 16, 4, False, 20, "invalid"),     # ids outside [0, E) are skipped
    (512, 256, 16, 4, True, 100, "uniform"),     # 400 pairs + 100 shared rows
    (512, 256, 1, 1, False, 16, "uniform"),      # one expert
    (512, 256, 16, 8, False, 65, "uniform"),     # 520 pairs: above the in-launch limit
    (512, 256, 300, 2, False, 20, "uniform"),    # E above the in-launch limit
    (2048, 768, 128, 8, False, 1, "uniform"),    # 8 rows: down + combine in one launch
    (1024, 2048, 32, 6, True, 2, "uniform"),     # 14 rows with the shared expert's, 16 slabs
    (512, 256, 16, 1, False, 1, "uniform"),      # one row
    (512, 256, 16, 2, True, 5, "hot"),           # 15 rows, a hot expert
]


def _pfc_ids(T, E, k, kind, seed):
    """Router-like ids [T][k] (distinct experts per token unless E < k)."""
    rng = np.random.default_rng(seed)
    if kind == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p = p[rng.permutation(E)]
        ids = np.stack([rng.choice(E, k, replace=False, p=p / p.sum()) for _ in range(T)])
    else:
        ids = np.stack([rng.permutation(E)[:k] if E >= k else rng.integers(0, E, k)
                        for _ in range(T)])
    if kind == "hot":
        for t in range(T):
            row = [e for e in ids[t] if e != 3][:k - 1]
            ids[t] = [3] + row if len(row) == k - 1 else ids[t]
    if kind == "invalid":
        m = rng.random((T, k)) < 0.15
        ids[m] = np.where(rng.random(m.sum()) < 0.5, -1, E)
    return ids.astype(np.int32)


@pytest.mark.parametrize("H,I,E,k,shared,T,kind", _PFC_CASES,
                         ids=[f"H{c[0]}-I{c[1]}-E{c[2]}-k{c[3]}{'-sh' if c[4] else ''}-T{c[5]}-{c[6]}"
                              for c in _PFC_CASES])
def test_permute_ffn_combine(lib, orc, H, I, E, k, shared, T, kind):
    """moe_permute_ffn_combine against moe_permute + moe_expert_ffn_combine on
    the same ids: offsets, sorted pairs, pair rows, y and the layer output bit
    for bit (the in-launch permutation is the same stable counting sort, and
    the FFN tiles compute the same sums); the permutation also against the
    oracle's; and whether the permutation launch ran (it must not where the
    gate/up launch derives the permutation)."""
    _announce(f"permute+ffn+combine: H={H} I={I} E={E} k={k} shared={shared} T={T} {kind}")
    cfg = synth.LayerConfig("pfc", H, E, k, I, "mxfp4", 1 if shared else 0, "uniform", (T,),
                            "gauss_mxfp4", seed=43)
    w = Workload(cfg)
    x = to_dev_bf16(synth.activations(cfg, T, step=2))
    ids_np = _pfc_ids(T, E, k, kind, seed=T * 7 + E)
    ids = torch.from_numpy(ids_np).to(DEV)
    wts = torch.from_numpy(np.random.default_rng(T).random((T, k), dtype=np.float32)).to(DEV)
    n = T * k
    rows = n + (T if shared else 0)
    _, fb = lib.moe_workspace_size(T, k + 1 if shared else k, H, I, E)
    sh_table = w.dev_shared.table if shared else None

    def bufs():
        return dict(off=torch.full((E + 1,), -5, dtype=torch.int32, device=DEV),
                    sp=torch.full((n,), -5, dtype=torch.int32, device=DEV),
                    pr=torch.full((n,), -5, dtype=torch.int32, device=DEV),
                    y=torch.zeros((rows, H), dtype=torch.bfloat16, device=DEV),
                    out=torch.zeros((T, H), dtype=torch.bfloat16, device=DEV),
                    ws=torch.empty(fb, dtype=torch.uint8, device=DEV))

    a = bufs()
    torch.cuda.synchronize()
    lib.moe_set_option(lib.MOE_OPT_TIMING, 1)
    lib.moe_permute_ffn_combine(x, ids, wts, w.dev.table, sh_table, lib.MOE_W_MXFP4, T, k, H, I,
                                E, a["off"], a["sp"], a["pr"], a["y"], a["out"], a["ws"], fb)
    torch.cuda.synchronize()
    launched = lib.timing_report()
    lib.moe_set_option(lib.MOE_OPT_TIMING, 0)
    b = bufs()
    lib.moe_permute(ids, T, k, E, b["off"], b["sp"], b["pr"], b["ws"], fb)
    lib.moe_expert_ffn_combine(x, b["sp"], b["off"], w.dev.table, sh_table, lib.MOE_W_MXFP4, T, k,
                               H, I, E, wts, b["y"], b["out"], b["ws"], fb)
    torch.cuda.synchronize()
    for name in ("off", "sp", "pr", "y", "out"):
        assert torch.equal(a[name], b[name]), f"{name} differs from the two calls"
    in_launch = n <= 512 and E <= 256
    perm_kernels = [kn for kn in launched if kn.startswith("permute")]
    if in_launch:
        assert not perm_kernels, f"permutation launched: {launched}"
    else:
        assert perm_kernels, f"no permutation launch: {launched}"
    if kind != "invalid":
        off_r, sp_r, pr_r = orc.permute(ids_np, E)
        assert np.array_equal(a["off"].cpu().numpy(), off_r)
        assert np.array_equal(a["sp"].cpu().numpy(), sp_r)
        assert np.array_equal(a["pr"].cpu().numpy(), pr_r)
    else:
        valid = (ids_np >= 0) & (ids_np < E)
        assert int(a["off"][E]) == int(valid.sum())
        assert (a["pr"].cpu().numpy().reshape(T, k)[~valid] == -5).all(), "skipped pairs written"
