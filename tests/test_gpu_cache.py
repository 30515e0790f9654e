"""GPU tests of the expert cache (LRU slots over pinned host blobs, device
table read by the expert FFN): slot bytes equal the host blob, the hit / miss
/ victim trace equals a brute-force LRU list, and outputs computed through the
cache equal the resident outputs bit for bit, also while the next layer's
experts stream in on the copy stream during the current layer's compute.

The pages' design keeps experts in host memory, loads them on demand and keeps
the frequently used ones in a global LRU cache, overlapping weight movement
with compute (winzheng.com page, "FreeToken's Three-Layer Mechanism")."""
from __future__ import annotations

import numpy as np
import pytest

from mixture_experts_gate_amd import synth

pytestmark = pytest.mark.gpu

# a small MXFP4 layer (kernel layout needs H, I multiples of 128)
H, I, E, K = 256, 256, 16, 4


def _blobs(n_layers, seed=11):
    cfg = synth.LayerConfig("cache_test", H, E, K, I, "mxfp4", 0, "uniform", (16,),
                            "gauss_mxfp4", layers=n_layers, seed=seed)
    return [synth.expert_pool(cfg, layer=l) for l in range(n_layers)]


@pytest.fixture(scope="module")
def env():
    import torch
    from mixture_experts_gate_amd import _lib
    from mixture_experts_gate_amd.layer import HostExperts, pack_to_device
    _lib.load()
    lay = synth.blob_layout(H, I, "mxfp4")
    L = 4
    blobs = _blobs(L)
    store = HostExperts(blobs, lay)
    resident = [pack_to_device(b, lay) for b in blobs]
    return dict(torch=torch, lib=_lib, lay=lay, L=L, blobs=blobs, store=store, resident=resident)


class LruModel:
    """Brute-force model of the cache policy: a list of slots from most to least
    recently used; a call hands out its hits first (ascending expert), then
    fills its misses (ascending expert) from the least recently used slot not
    handed out by the same call."""

    def __init__(self, nslots, E):
        self.order = list(reversed(range(nslots)))      # free slots: lowest index taken first
        self.key_of = [-1] * nslots
        self.slot_of = {}
        self.last = [0] * nslots
        self.gen = 0
        self.E = E
        self.hits = self.misses = 0

    def _front(self, s):
        self.order.remove(s)
        self.order.insert(0, s)

    def prefetch(self, layer, ids):
        want = sorted(set(int(i) for i in ids)) if ids is not None else list(range(self.E))
        self.gen += 1
        g = self.gen
        miss = []
        for e in want:
            s = self.slot_of.get(layer * self.E + e, -1)
            if s >= 0:
                self.hits += 1
                self._front(s)
                self.last[s] = g
            else:
                miss.append(e)
        for e in miss:
            s = next(s for s in reversed(self.order) if self.last[s] != g)
            if self.key_of[s] >= 0:
                del self.slot_of[self.key_of[s]]
            key = layer * self.E + e
            self.key_of[s] = key
            self.slot_of[key] = s
            self._front(s)
            self.last[s] = g
            self.misses += 1

    def resize(self, n2, same_pool):
        """Keep the n2 most recently used residents: a kept slot below n2 stays,
        the others take the lowest free indices (most recent first); free slots
        follow at the least recently used end, the lowest index last (taken
        first)."""
        res = [s for s in self.order if self.key_of[s] >= 0]
        kept, dropped = res[:n2], res[n2:]
        for s in dropped:
            del self.slot_of[self.key_of[s]]
        used = [False] * n2
        for s in kept:
            if s < n2:
                used[s] = True
        dst, f = [], 0
        for s in kept:
            if s < n2:
                dst.append(s)
            else:
                while used[f]:
                    f += 1
                used[f] = True
                dst.append(f)
        key2 = [-1] * n2
        for s, d in zip(kept, dst):
            key2[d] = self.key_of[s]
        self.key_of = key2
        self.slot_of = {k: d for d, k in enumerate(key2) if k >= 0}
        self.order = dst + [s for s in reversed(range(n2)) if not used[s]]
        self.last = [0] * n2
        return sum(1 for s, d in zip(kept, dst) if s != d or not same_pool)

    def evict(self, layer, ids):
        for e in (ids if ids is not None else range(self.E)):
            s = self.slot_of.pop(layer * self.E + int(e), None)
            if s is not None:
                self.key_of[s] = -1
                self.order.remove(s)
                self.order.append(s)


def _cache(env, nslots):
    from mixture_experts_gate_amd.layer import ExpertCache
    slot = (env["lay"].nbytes + 255) // 256 * 256
    return ExpertCache(env["store"], env["L"], E, nslots * slot)


def test_prefetched_slots_hold_the_host_bytes(env):
    torch = env["torch"]
    c = _cache(env, 24)
    try:
        c.prefetch(1, np.array([3, 5, 7, 3]))
        c.prefetch(2, None)
        torch.cuda.synchronize()
        nb = env["lay"].nbytes
        checked = 0
        for l in range(env["L"]):
            for e in range(E):
                s = c.slot_of(l, e)
                if s < 0:
                    continue
                got = c.slot_bytes_view(s, nb).cpu()
                want = env["store"].host[l * E + e]
                assert torch.equal(got, want), (l, e, s)
                checked += 1
        assert checked == 3 + E           # 24 slots hold both requests
        h, m, b = c.stats()
        assert b == m * nb
    finally:
        c.close()


def test_lru_trace_matches_brute_force(env):
    torch = env["torch"]
    nslots = 20
    c = _cache(env, nslots)
    model = LruModel(nslots, E)
    rng = np.random.default_rng(5)
    try:
        for step in range(80):
            layer = int(rng.integers(env["L"]))
            if step % 17 == 16:
                ids = rng.choice(E, size=int(rng.integers(1, 5)), replace=False)
                c.evict(layer, ids)
                model.evict(layer, ids)
                continue
            if step % 23 == 0:
                ids = None
            else:
                ids = rng.integers(0, E, size=int(rng.integers(1, 12)))
            c.prefetch(layer, ids)
            model.prefetch(layer, ids)
            for l in range(env["L"]):
                for e in range(E):
                    assert c.slot_of(l, e) == model.slot_of.get(l * E + e, -1), (step, l, e)
            h, m, _ = c.stats()
            assert (h, m) == (model.hits, model.misses), step
        torch.cuda.synchronize()
    finally:
        c.close()


def test_bad_request_changes_nothing(env):
    lib = env["lib"]
    c = _cache(env, E)          # exactly one layer fits
    try:
        c.prefetch(0, None)
        before = [c.slot_of(0, e) for e in range(E)]
        stats = c.stats()
        for bad in (np.array([1, 2, E]), np.array([-1])):
            with pytest.raises(lib.MoeError):
                c.prefetch(1, bad)
        with pytest.raises(lib.MoeError):
            c.prefetch(env["L"], None)
        assert [c.slot_of(0, e) for e in range(E)] == before
        assert c.stats() == stats
        # with room for one layer only, the next layer takes every slot over
        c.prefetch(1, None)
        assert sorted(c.slot_of(1, e) for e in range(E)) == sorted(before)
        assert all(c.slot_of(0, e) == -1 for e in range(E))
    finally:
        c.close()


def _layer_outputs(env, tables, T, seed):
    """Run the FFN of every layer with its table; returns y per layer (host)."""
    import torch
    from mixture_experts_gate_amd.layer import MoeLayer
    out = []
    rng = np.random.default_rng(seed)
    L = MoeLayer(H, E, K, I, "mxfp4", T)
    x = torch.from_numpy(
        synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)).view(np.int16)
    ).cuda()
    logits = torch.from_numpy(rng.random((T, E), dtype=np.float32)).cuda()
    L.route_permute(T, logits=logits, write_logits=False)
    for tab in tables:
        L.ffn(T, x, tab)
        out.append(L.y[:T * K].clone())
    torch.cuda.synchronize()
    return [o.cpu() for o in out]


@pytest.mark.parametrize("T", [8, 512])
def test_cached_output_equals_resident_bitwise(env, T):
    torch = env["torch"]
    from mixture_experts_gate_amd.layer import expert_table
    lay = env["lay"]
    res_tabs = [expert_table(r.data_ptr(), E, lay) for r in env["resident"]]
    want = _layer_outputs(env, res_tabs, T, seed=T)
    c = _cache(env, 2 * E)
    try:
        tabs = []
        for l in range(env["L"]):
            tabs.append(c.prefetch(l, None))
            torch.cuda.synchronize()      # each table used before the next call refills slots
            got = _layer_outputs(env, [tabs[-1]], T, seed=T)[0]
            assert torch.equal(got, want[l]), l
    finally:
        c.close()


def test_streaming_next_layer_during_compute_is_bitwise(env):
    """Double-buffered stack: prefetch(l + 1) is called right after layer l's
    compute is enqueued, so its copies run while layer l computes and reuse the
    slots of layer l - 1. Outputs of three passes over the 4-layer stack equal
    the resident outputs bit for bit."""
    torch = env["torch"]
    from mixture_experts_gate_amd.layer import MoeLayer, expert_table
    lay = env["lay"]
    T = 512
    res_tabs = [expert_table(r.data_ptr(), E, lay) for r in env["resident"]]
    want = _layer_outputs(env, res_tabs, T, seed=77)
    rng = np.random.default_rng(77)
    Lyr = MoeLayer(H, E, K, I, "mxfp4", T)
    x = torch.from_numpy(
        synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)).view(np.int16)
    ).cuda()
    logits = torch.from_numpy(rng.random((T, E), dtype=np.float32)).cuda()
    Lyr.route_permute(T, logits=logits, write_logits=False)
    c = _cache(env, 2 * E)
    outs = []
    try:
        tab = c.prefetch(0, None)
        for step in range(3 * env["L"]):
            l = step % env["L"]
            Lyr.ffn(T, x, tab)
            outs.append((l, Lyr.y[:T * K].clone()))
            tab = c.prefetch((l + 1) % env["L"], None)
        torch.cuda.synchronize()
        for l, y in outs:
            assert torch.equal(y.cpu(), want[l]), l
        h, m, b = c.stats()
        assert m >= 3 * env["L"] * E - E     # every layer change misses (two layers fit)
    finally:
        c.close()


def test_resize_trace_matches_brute_force(env):
    """Prefetches, evictions and resizes (shrink and grow, in place and into a
    new pool) against the model; after each resize the residents' slots hold
    the host bytes, so nothing had to be reloaded."""
    torch = env["torch"]
    nb = env["lay"].nbytes
    slot = (nb + 255) // 256 * 256
    c = _cache(env, 30)
    model = LruModel(30, E)
    rng = np.random.default_rng(8)
    sizes = [(20, True), (34, False), (16, False), (26, True), (40, False), (E, True)]
    try:
        for step in range(60):
            layer = int(rng.integers(env["L"]))
            if step % 10 == 9:
                n2, inplace = sizes[(step // 10) % len(sizes)]
                if inplace and n2 * slot > c.pool.numel():
                    inplace = False
                h0, m0, b0 = c.stats()
                moved = c.resize(n2 * slot, in_place=inplace)
                want_moved = model.resize(n2, inplace)
                assert moved == want_moved, step
                assert c.slots() == n2
                assert c.stats() == (h0, m0, b0)        # no host traffic
                torch.cuda.synchronize()
                for l in range(env["L"]):
                    for e in range(E):
                        s = c.slot_of(l, e)
                        assert s == model.slot_of.get(l * E + e, -1), (step, l, e)
                        if s >= 0:
                            got = c.slot_bytes_view(s, nb).cpu()
                            assert torch.equal(got, env["store"].host[l * E + e]), (step, l, e)
                continue
            ids = None if step % 7 == 0 else rng.integers(0, E, size=int(rng.integers(1, 12)))
            c.prefetch(layer, ids)
            model.prefetch(layer, ids)
            if step % 13 == 12:
                ev = rng.choice(E, size=2, replace=False)
                c.evict(layer, ev)
                model.evict(layer, ev)
            for l in range(env["L"]):
                for e in range(E):
                    assert c.slot_of(l, e) == model.slot_of.get(l * E + e, -1), (step, l, e)
            assert c.stats()[:2] == (model.hits, model.misses), step
        torch.cuda.synchronize()
    finally:
        c.close()


def test_resize_between_layers_is_bitwise(env):
    """Stack passes with the pool shrunk to one layer and grown back in between:
    outputs equal the resident outputs bit for bit, and the residents kept by a
    resize are hits afterwards."""
    torch = env["torch"]
    from mixture_experts_gate_amd.layer import expert_table
    lay = env["lay"]
    slot = (lay.nbytes + 255) // 256 * 256
    T = 64
    res_tabs = [expert_table(r.data_ptr(), E, lay) for r in env["resident"]]
    want = _layer_outputs(env, res_tabs, T, seed=31)
    c = _cache(env, 3 * E)
    try:
        for step in range(2 * env["L"]):
            l = step % env["L"]
            if step == 3:
                c.resize(E * slot)                      # one layer's worth, new pool
            if step == 5:
                c.resize(3 * E * slot)                  # grow back, new pool
            if step == 6:
                c.resize(2 * E * slot, in_place=True)   # shrink in place
            tab = c.prefetch(l, None)
            got = _layer_outputs(env, [tab], T, seed=31)[0]
            torch.cuda.synchronize()
            assert torch.equal(got, want[l]), (step, l)
        # the layer used right before a resize stays resident through it
        c.prefetch(1, None)
        before = c.stats()
        c.resize(E * slot)
        c.prefetch(1, None)
        after = c.stats()
        assert after[1] == before[1] and after[0] == before[0] + E
    finally:
        c.close()


def test_resize_errors_leave_the_cache_unchanged(env):
    """A pool with fewer slots than one layer's experts is refused (ENOMEM), and
    so is a new pool that partly overlaps the current one (EINVAL); neither
    changes the slots, the counters or the residents' bytes."""
    torch = env["torch"]
    lib = env["lib"]
    nb = env["lay"].nbytes
    slot = (nb + 255) // 256 * 256
    c = _cache(env, 2 * E)
    try:
        c.prefetch(0, None)
        c.prefetch(1, np.arange(5))
        torch.cuda.synchronize()
        before = [[c.slot_of(l, e) for e in range(E)] for l in range(env["L"])]
        stats = c.stats()
        with pytest.raises(lib.MoeError) as ei:
            c.resize((E - 1) * slot)
        assert ei.value.code == lib.MOE_ENOMEM
        overlap = c.pool.data_ptr() + slot            # starts inside the current pool
        with pytest.raises(lib.MoeError) as ei:
            lib.expert_cache_resize(c.handle, overlap, E * slot)
        assert ei.value.code == lib.MOE_EINVAL
        assert [[c.slot_of(l, e) for e in range(E)] for l in range(env["L"])] == before
        assert c.stats() == stats and c.slots() == 2 * E
        for l in range(env["L"]):
            for e in range(E):
                s = c.slot_of(l, e)
                if s >= 0:
                    assert torch.equal(c.slot_bytes_view(s, nb).cpu(), env["store"].host[l * E + e])
    finally:
        c.close()


# ------------------------------------------------------------ fault injection --

def _slots_all(c, env):
    return [[c.slot_of(l, e) for e in range(E)] for l in range(env["L"])]


def test_injected_copy_failure_leaves_cache_unchanged(env):
    """A copy that fails at the first copy of a call (injected: not issued)
    returns MOE_EHIP and leaves slots, LRU order and counters as they were;
    the trace afterwards still matches the brute-force LRU model. A failure
    at the third copy keeps exactly the two misses copied before it (their
    bytes arrive), and a retry of the same request completes the layer."""
    torch, lib = env["torch"], env["lib"]
    nb = env["lay"].nbytes
    nslots = 2 * E
    c = _cache(env, nslots)
    model = LruModel(nslots, E)
    try:
        for l, ids in ((0, None), (1, np.array([2, 9, 4])), (2, np.arange(10))):
            c.prefetch(l, ids)
            model.prefetch(l, ids)
        torch.cuda.synchronize()
        before, stats = _slots_all(c, env), c.stats()
        lib.moe_set_option(lib.MOE_OPT_CACHE_FAULT, 1)
        with pytest.raises(lib.MoeError) as ei:
            c.prefetch(3, np.array([1, 5, 6]))          # three misses
        assert ei.value.code == lib.MOE_EHIP
        lib.moe_set_option(lib.MOE_OPT_CACHE_FAULT, 1)
        with pytest.raises(lib.MoeError):
            c.prefetch(2, np.arange(8, 16))             # hits of layer 2 and misses
        assert lib.moe_get_option(lib.MOE_OPT_CACHE_FAULT) == 0     # the knob fired
        assert _slots_all(c, env) == before and c.stats() == stats
        # the failed calls changed nothing the model does not know about
        rng = np.random.default_rng(3)
        for step in range(30):
            layer = int(rng.integers(env["L"]))
            ids = None if step % 9 == 0 else rng.integers(0, E, size=int(rng.integers(1, 9)))
            c.prefetch(layer, ids)
            model.prefetch(layer, ids)
            assert _slots_all(c, env) == [[model.slot_of.get(l * E + e, -1) for e in range(E)]
                                          for l in range(env["L"])], step
            assert c.stats()[:2] == (model.hits, model.misses)
        # partial failure: the third copy of the call fails
        c.evict(3, None)
        model.evict(3, None)
        h0, m0, _ = c.stats()
        lib.moe_set_option(lib.MOE_OPT_CACHE_FAULT, 3)
        with pytest.raises(lib.MoeError) as ei:
            c.prefetch(3, np.arange(6))
        assert ei.value.code == lib.MOE_EHIP
        torch.cuda.synchronize()
        got = [c.slot_of(3, e) for e in range(6)]
        assert all(s >= 0 for s in got[:2]) and all(s == -1 for s in got[2:]), got
        assert c.stats()[:2] == (h0, m0 + 2)
        for e in range(2):
            assert torch.equal(c.slot_bytes_view(got[e], nb).cpu(), env["store"].host[3 * E + e])
        c.prefetch(3, np.arange(6))
        h1, m1, _ = c.stats()
        assert (h1, m1) == (h0 + 2, m0 + 6)
        torch.cuda.synchronize()
        for e in range(6):
            s = c.slot_of(3, e)
            assert torch.equal(c.slot_bytes_view(s, nb).cpu(), env["store"].host[3 * E + e])
    finally:
        lib.moe_set_option(lib.MOE_OPT_CACHE_FAULT, 0)
        c.close()


def _stream_stack(env, c, T, passes, seed):
    """Double-buffered pass over the stack through cache c: layer l+1 is
    requested right after layer l's FFN is enqueued. Returns [(layer, y)]."""
    torch = env["torch"]
    from mixture_experts_gate_amd.layer import MoeLayer
    rng = np.random.default_rng(seed)
    Lyr = MoeLayer(H, E, K, I, "mxfp4", T)
    x = torch.from_numpy(
        synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32)).view(np.int16)
    ).cuda()
    logits = torch.from_numpy(rng.random((T, E), dtype=np.float32)).cuda()
    Lyr.route_permute(T, logits=logits, write_logits=False)
    outs = []
    tab = c.prefetch(0, None)
    for step in range(passes * env["L"]):
        l = step % env["L"]
        Lyr.ffn(T, x, tab)
        outs.append((l, Lyr.y[:T * K].clone()))
        tab = c.prefetch((l + 1) % env["L"], None)
    torch.cuda.synchronize()
    return outs


def test_delayed_copy_stream_is_bitwise(env):
    """Every prefetch's copies held back 20 ms on the copy stream (a slow
    link): the compute of each layer still waits for its own copies and never
    reads a slot being refilled, so the streamed outputs equal the resident
    ones bit for bit."""
    torch, lib = env["torch"], env["lib"]
    from mixture_experts_gate_amd.layer import expert_table
    lay = env["lay"]
    T = 256
    res_tabs = [expert_table(r.data_ptr(), E, lay) for r in env["resident"]]
    want = _layer_outputs(env, res_tabs, T, seed=19)
    c = _cache(env, 2 * E)
    lib.moe_set_option(lib.MOE_OPT_CACHE_DELAY_US, 20000)
    try:
        outs = _stream_stack(env, c, T, 2, seed=19)
    finally:
        lib.moe_set_option(lib.MOE_OPT_CACHE_DELAY_US, 0)
        c.close()
    for l, y in outs:
        assert torch.equal(y.cpu(), want[l]), l


def test_thrash_at_one_layer_capacity_is_bitwise(env):
    """A pool of exactly one layer of experts: every request of the next layer
    replaces every slot (each waits for the previous layer's compute), all
    misses, and the outputs equal the resident ones bit for bit."""
    torch = env["torch"]
    from mixture_experts_gate_amd.layer import expert_table
    lay = env["lay"]
    T = 64
    res_tabs = [expert_table(r.data_ptr(), E, lay) for r in env["resident"]]
    want = _layer_outputs(env, res_tabs, T, seed=23)
    c = _cache(env, E)
    try:
        outs = _stream_stack(env, c, T, 3, seed=23)
        h, m, _ = c.stats()
        assert h == 0 and m == (3 * env["L"] + 1) * E
    finally:
        c.close()
    for l, y in outs:
        assert torch.equal(y.cpu(), want[l]), l


# ------------------------------------------------- bandwidth-adaptive choice --

def test_bandwidth_is_measured(env):
    """The cache's rate comes from events around its copies: positive after a
    completed copy, and close to the forced rate when the link is throttled."""
    torch, lib = env["torch"], env["lib"]
    c = _cache(env, 2 * E)
    try:
        assert c.bandwidth() == (0.0, 0)
        c.prefetch(0, None)
        torch.cuda.synchronize()
        g, n = c.bandwidth()
        assert n == 1 and g > 0.2, (g, n)
    finally:
        c.close()
    c = _cache(env, 2 * E)
    lib.moe_set_option(lib.MOE_OPT_CACHE_THROTTLE_MBS, 200)
    try:
        c.prefetch(1, None)
        torch.cuda.synchronize()
        g, n = c.bandwidth()
        assert n == 1 and 0.05 < g < 0.21, g          # 1 / (1/0.2 + 1/link) GB/s
    finally:
        lib.moe_set_option(lib.MOE_OPT_CACHE_THROTTLE_MBS, 0)
        c.close()


@pytest.mark.parametrize("mode", ["host", "device", "mixed"])
def test_qstar_layer_matches_oracle(env, orc, mode):
    """A layer through the cache with the bandwidth-adaptive choice. "host":
    free host time, every miss is computed on the host CPU; "device": costly
    host time, every miss is copied; "mixed": host time close to the copy time,
    some of each. Routing and the layer output against the oracle; the host
    experts' rows against the oracle's rows; with no host expert, the output
    equals the resident layer's bit for bit."""
    torch = env["torch"]
    from mixture_experts_gate_amd.layer import MoeLayer, expert_table
    from parity import assert_close, bf16_dev_to_f64
    lay = env["lay"]
    T, l = 12, 2
    rng = np.random.default_rng(7)
    x_bits = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    lg = rng.random((T, E), dtype=np.float32)
    x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
    lgd = torch.from_numpy(lg).cuda()
    costs = {"host": (0.0, 0.0, 1.0), "device": (1.0, 1.0, 1e6), "mixed": (90e-6, 0.0, 1.0)}[mode]
    c = _cache(env, 2 * E)
    Lq = MoeLayer(H, E, K, I, "mxfp4", T)
    try:
        out, mask = Lq.forward_cached_qstar(T, x, c, l, logits=lgd, host_s_per_expert=costs[0],
                                            host_s_per_row=costs[1], link_gbs=costs[2], threads=4)
        torch.cuda.synchronize()
        used = np.unique(Lq.topk_ids[:T].cpu().numpy())
        nh = int(mask.sum())
        if mode == "host":
            assert nh == len(used)
        elif mode == "device":
            assert nh == 0
        else:
            assert 0 < nh < len(used), nh
        for e in range(E):
            assert (c.slot_of(l, e) >= 0) == (e in used and not mask[e]), e
        ref = orc.moe_layer(x_bits, lay, env["blobs"][l], K, logits=lg)
        assert np.array_equal(Lq.topk_ids[:T].cpu().numpy(), ref["ids"])
        assert_close(bf16_dev_to_f64(out), ref["out_f64"], f"q* layer output ({mode})")
        y = Lq.y[:T * K].float().cpu().numpy().astype(np.float64)
        pairs = np.nonzero(mask[ref["ids"].ravel()])[0]
        if len(pairs):
            assert_close(y[pairs], ref["y"][pairs], f"host expert rows ({mode})")
        if nh == 0:
            res = expert_table(env["resident"][l].data_ptr(), E, lay)
            Lr = MoeLayer(H, E, K, I, "mxfp4", T)
            out_r = Lr.forward(T, x, res, logits=lgd)
            torch.cuda.synchronize()
            assert torch.equal(out, out_r)
    finally:
        c.close()


def test_qstar_live_host_cost(env, orc):
    """q* with the host's cost per expert measured live: after a layer whose
    misses ran on the host (a zero seed), the cache holds a positive
    per-expert time, the next layer's choice uses it in place of the seed, and
    both layers' outputs match the oracle."""
    torch = env["torch"]
    from mixture_experts_gate_amd.layer import MoeLayer
    from parity import assert_close, bf16_dev_to_f64
    lay = env["lay"]
    T = 12
    rng = np.random.default_rng(9)
    c = _cache(env, 2 * E)
    Lq = MoeLayer(H, E, K, I, "mxfp4", T)
    try:
        assert c.host_s_per_expert_live is None
        for l in (1, 3):
            x_bits = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
            lg = rng.random((T, E), dtype=np.float32)
            x = torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)
            out, mask = Lq.forward_cached_qstar(T, x, c, l, logits=torch.from_numpy(lg).cuda(),
                                                host_s_per_expert=0.0, host_s_per_row=0.0,
                                                link_gbs=1.0, threads=4, live_host=True)
            torch.cuda.synchronize()
            if l == 1:
                assert mask.sum() > 0        # free host time: every miss on the host
            live = c.host_s_per_expert_live
            assert live is not None and 0.0 < live < 1.0, live
            ref = orc.moe_layer(x_bits, lay, env["blobs"][l], K, logits=lg)
            assert np.array_equal(Lq.topk_ids[:T].cpu().numpy(), ref["ids"])
            assert_close(bf16_dev_to_f64(out), ref["out_f64"], f"q* live layer {l}")
    finally:
        c.close()
