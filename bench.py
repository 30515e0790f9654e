#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X.

One step = one pass of the routed MoE expert layer (route -> permute ->
grouped SwiGLU expert FFN -> combine) over one batch of synthetic tokens, all
inputs resident in HBM. The headline workload is the decode-shaped layer
(H=2048, 128 experts, top-8, I=768, MXFP4 weights, bf16 activations, uniform
router logits) at T=64 tokens. The JSON line's sweep also carries T=1, 8, 32
and the prefill-shaped T=8192 batch of the same layer; the large sparse layer
(H=4096, 256 experts + 1 shared, top-6, I=2048, Zipf popularity) at T=1, 64,
4096; and the 43-layer stack of that layer decoding T=1, 2, 4, 8 and 16 tokens,
once with every layer resident in HBM and once through a 32 GB LRU expert
cache fed from pinned host memory (hit rate, H2D bytes and GB/s against the
measured pinned copy rate; T=1 over 1024 steps, four popularity phases);
full-layer double-buffered prefill streaming of that stack at T=4096 (time
per layer against the copy alone and the compute alone); references measured
on the GPU (read stream at the kernels' byte counts, matrix-core issue rates).

Timing: W eager warm-up steps, then K steps replayed from HIP graphs (one
graph holds 16 consecutive steps), bracketed by device synchronisation.
Steps rotate over 8 replicas of the expert weights (8 x 321 MB, well above the
256 MB last-level cache) and 8 input batches, so weight bytes come from HBM.

roofline: the dominant kernel's algorithmic bytes per launch divided by its
average launch time, from the start/end events hipExtLaunchKernel attaches to
each of its dispatches on the launch stream (library timing mode, a second
pass of K eager steps); traffic: HBM bytes per launch from the committed
counter summary (profiles/traffic.json) when it matches the kernel's source.
cpu_baseline: the CPU oracle (single-threaded C, fp64) on the same layer;
cpu_baseline_sweep: the oracle on every workload (token subsets of the large
batches, extrapolation labelled), with the host's CPU model.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak, published
REPLICAS = 8
STEPS_PER_GRAPH = 16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--T", type=int, default=64)
    ap.add_argument("--no-sweep", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--profile", action="store_true",
                    help="short run for profilers: headline workload, no sweep, no CPU leg")
    ap.add_argument("--no-stack", action="store_true", help="skip the 43-layer stack runs")
    ap.add_argument("--only", default="",
                    help="comma list of sweep parts to run: "
                         "decode,formats,prefill,cfg4,stack,stream,qstar")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 512 MiB device copy (HBM counter calibration)")
    ap.add_argument("--no-micro", action="store_true",
                    help="skip the read-stream / matrix-core reference measurements")
    ap.add_argument("--stack-steps", type=int, default=1024,
                    help="timed steps of the cached 43-layer stack at T=1")
    ap.add_argument("--cfg4-T", default="1,2,64,4096",
                    help="comma list of the large sparse layer's batch sizes to run")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "ffn_decode_gate_up": ["mixture_experts_gate_amd/csrc/ffn_decode.hip",
                           "mixture_experts_gate_amd/csrc/common.hpp"],
    "ffn_decode_down": ["mixture_experts_gate_amd/csrc/ffn_decode.hip",
                        "mixture_experts_gate_amd/csrc/common.hpp"],
    "ffn_prefill_gate_up": ["mixture_experts_gate_amd/csrc/ffn_prefill.hip",
                            "mixture_experts_gate_amd/csrc/common.hpp"],
    "ffn_prefill_down": ["mixture_experts_gate_amd/csrc/ffn_prefill.hip",
                         "mixture_experts_gate_amd/csrc/common.hpp"],
}


def measured_traffic(kernel, T):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current source of the kernel (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(f"{kernel}@T={T}")
    if not rec or rec.get("source_digest") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


class Workload:
    """One routed MoE layer of config ``cfg`` at T tokens, inputs resident in
    HBM: ``replicas`` copies of the expert weights and ``batches`` input
    batches (default: as many as replicas, 64 at T <= 8 so that a cycle of
    steps touches several times the 256 MB last-level cache even when each
    step touches few experts), step i using replica i mod R and batch i mod B
    (plus the shared expert when the config has one)."""

    def __init__(self, torch, cfg, T, dev, replicas=REPLICAS, pool=None, dexp=None,
                 shared=None, batches=None):
        from mixture_experts_gate_amd import synth
        from mixture_experts_gate_amd.layer import DeviceExperts, MoeLayer
        self.cfg = c = cfg
        self.T = T
        self.lay = synth.blob_layout(c.H, c.I, c.fmt)
        self.pool = synth.expert_pool(c) if pool is None else pool
        self.dexp = DeviceExperts(self.pool, self.lay, copies=replicas, device=dev) if dexp is None else dexp
        self.R = len(self.dexp.tables)
        self.has_shared = c.n_shared > 0
        self.sh = None
        if self.has_shared:
            self.sh = shared if shared is not None else DeviceExperts(
                synth.shared_expert(c)[None, :], self.lay, copies=self.R, device=dev)
        to16 = lambda a: torch.from_numpy(a.view("int16")).to(dev)
        self.B = batches if batches is not None else (64 if T <= 8 else self.R)
        self.x_host = [synth.activations(c, T, step=r) for r in range(self.B)]
        self.lg_host = [synth.router_logits(c, T, step=r) for r in range(self.B)]
        self.x = [to16(a) for a in self.x_host]
        self.lg = [torch.from_numpy(a).to(dev) for a in self.lg_host]
        self.layer = MoeLayer(c.H, c.E, c.k, c.I, c.fmt, T, shared=self.has_shared, device=dev)
        self.fuse_shared = True
        if self.has_shared:
            self.layer.prepare_shared(T)

    def step(self, i):
        r, b = i % self.R, i % self.B
        self.layer.forward(self.T, self.x[b], self.dexp.tables[r], logits=self.lg[b],
                           shared_table=self.sh.tables[r] if self.has_shared else None,
                           fuse_shared=self.fuse_shared)

    def unique_experts(self, torch):
        """Distinct experts the GPU router picks per step (average over the input
        batches), read back from its top-k ids."""
        import numpy as np
        us = []
        for r in range(self.B):
            self.layer.route(self.T, logits=self.lg[r], write_logits=False)
            torch.cuda.synchronize()
            us.append(len(np.unique(self.layer.topk_ids[:self.T].cpu().numpy())))
        return float(np.mean(us)), us


WARM_REPLAY_STEPS = [0]     # untimed graph-replayed steps of the last time_graphs call


def time_graphs(torch, wl, steps, warmup):
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    n_graph = min(STEPS_PER_GRAPH, steps)
    graphs = []
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_graph):
            wl.step(i)
    graphs.append((g, n_graph))
    rem = steps % n_graph
    if rem:
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2):
            for i in range(rem):
                wl.step(i)
        graphs.append((g2, rem))
    # warm replays (untimed): every graph once, so that no graph's first
    # replay is timed, then the full graph again until about 20 ms of device
    # work have run, so that the timed replays start at working clocks (after
    # the host-side setup the device has idled)
    for g_, _ in graphs:
        g_.replay()
    torch.cuda.synchronize()
    warm_steps = sum(n for _, n in graphs)
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < 0.02:
        graphs[0][0].replay()
        torch.cuda.synchronize()
        warm_steps += n_graph
    WARM_REPLAY_STEPS[0] = warm_steps
    reps = steps // n_graph
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(reps):
        graphs[0][0].replay()
    if rem:
        graphs[1][0].replay()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop)
    del graphs
    return ms, wall


def kernel_timing(torch, wl, steps):
    """Average dispatch time of each kernel over `steps` eager steps, each step
    run on an idle device (synchronised after it), so that no dispatch's window
    also covers queued work from another step."""
    from mixture_experts_gate_amd import _lib
    torch.cuda.synchronize()
    _lib.moe_set_option(_lib.MOE_OPT_TIMING, 1)
    for i in range(steps):
        wl.step(i)
        torch.cuda.synchronize()
    rep = _lib.timing_report()
    _lib.moe_set_option(_lib.MOE_OPT_TIMING, 0)
    return {k: {"launches": n, "avg_us": 1000.0 * ms / n} for k, (n, ms) in rep.items()}


def algorithmic_bytes(wl, U):
    """Bytes each kernel must move at minimum (weights of touched experts read
    once, activations read once, outputs written once). With a shared expert
    the layer adds its weights and its output; the per-kernel figures are those
    of one step: with a shared expert, the FFN kernels run once for the routed
    experts and once for the shared one, and their figures cover both."""
    c, T, lay = wl.cfg, wl.T, wl.lay
    H, I, E, k = c.H, c.I, c.E, c.k
    w13 = lay.w2 - lay.w13           # W13 codes + scales of one expert
    w2 = lay.nbytes - lay.w2         # W2 codes + scales
    n = T * k
    sh = (lay.nbytes + T * H * 2) if c.n_shared else 0
    s13 = (w13 + T * H * 2 + T * I * 2) if c.n_shared else 0
    s2 = (w2 + T * I * 2 + T * H * 2) if c.n_shared else 0
    return {
        "route": T * E * 4 + n * 8,
        "permute_small": n * 4 + n * 8 + (E + 1) * 4,
        "ffn_decode_gate_up": U * w13 + T * H * 2 + n * I * 2 + s13,
        "ffn_decode_down": U * w2 + n * I * 2 + n * H * 2 + s2,
        "ffn_prefill_gate_up": U * w13 + T * H * 2 + n * I * 2 + s13,
        "ffn_prefill_down": U * w2 + n * I * 2 + n * H * 2 + s2,
        "combine": n * H * 2 + n * 4 + T * H * 2 + (T * H * 2 if c.n_shared else 0),
        "layer": U * lay.nbytes + 2 * T * H * 2 + T * E * 4 + n * 8 + sh,
        # the one-launch layer moves the whole layer's bytes
        "layer_fused": U * lay.nbytes + 2 * T * H * 2 + T * E * 4 + n * 8 + sh,
    }


def run_workload(torch, cfg, T, steps, warmup, dev, pool=None, dexp=None, shared=None,
                 kernel_steps=None, replicas=REPLICAS):
    wl = Workload(torch, cfg, T, dev, replicas=replicas, pool=pool, dexp=dexp, shared=shared)
    U, _ = wl.unique_experts(torch)
    ms, wall = time_graphs(torch, wl, steps, warmup)
    kt = kernel_timing(torch, wl, kernel_steps or min(steps, 64))
    ab = algorithmic_bytes(wl, U)
    ms_step = ms / steps
    c = wl.cfg
    flops = 6.0 * c.H * c.I * T * (c.k + c.n_shared)
    res = {
        "config": c.name,
        "T": T,
        "tokens_per_s": T * steps / (ms / 1000.0),
        "ms_per_step": ms_step,
        "host_wall_ms_per_step": 1000.0 * wall / steps,
        "warm_replay_steps": WARM_REPLAY_STEPS[0],
        "unique_experts": U,
        "layer_algorithmic_bytes": ab["layer"],
        "layer_hbm_GBs": ab["layer"] / (ms_step / 1000.0) / 1e9,
        "layer_hbm_frac": ab["layer"] / (ms_step / 1000.0) / 1e9 / HBM_PEAK_GBS,
        "layer_tflops": flops / (ms_step / 1000.0) / 1e12,
        "kernels": kt,
    }
    ksteps = kernel_steps or min(steps, 64)
    for name, v in kt.items():
        # per step: the launches of one step together move ab[name] bytes
        v["us_per_step"] = v["avg_us"] * v["launches"] / ksteps
        if name in ab:
            v["algorithmic_bytes"] = ab[name]
            v["GBs"] = ab[name] / (v["us_per_step"] * 1e-6) / 1e9
    return wl, res


def roofline(res, T):
    kt = res["kernels"]
    dom = max(kt, key=lambda n: kt[n]["launches"] and kt[n]["avg_us"] * kt[n]["launches"])
    k = kt[dom]
    if dom.startswith("ffn_prefill"):
        # the prefill contraction is matrix-core bound: FLOPs of this kernel
        return dom, {"bound": "mfma", "kernel": dom, "avg_us": k["avg_us"],
                     "unit": "TFLOP/s", "peak": BF16_PEAK_TFLOPS, "achieved": None,
                     "frac": None, "traffic": measured_traffic(dom, T)}
    ach = k.get("GBs")
    return dom, {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": None if ach is None else ach / HBM_PEAK_GBS,
                 "traffic": measured_traffic(dom, T),
                 "algorithmic_bytes_per_launch": k.get("algorithmic_bytes"),
                 "avg_us": k["avg_us"], "launches": k["launches"],
                 "timing": "hipExtLaunchKernel start/end events of each launch, K eager steps"}


class Stack:
    """The 43-layer stack of config-4-shaped layers (config 5): layer l's bf16
    output is layer l+1's input; each layer has its own router logits (Zipf
    popularity re-permuted every 256 steps) and its shared expert.

    Weights: ``distinct`` layers are generated (the remaining layers repeat
    them with that period); in the resident run every one of the 43 layers
    has its own full copy in HBM, so a step reads the same bytes it would with
    43 distinct layers."""

    def __init__(self, torch, cfg, dev, distinct=2):
        from mixture_experts_gate_amd import synth
        self.cfg = c = cfg
        self.L = c.layers
        self.D = distinct
        self.lay = synth.blob_layout(c.H, c.I, c.fmt)
        self.blobs = [synth.expert_pool(c, layer=d) for d in range(distinct)]
        self.shared_blobs = [synth.shared_expert(c, layer=d) for d in range(distinct)]
        self.dev = dev

    def host_store(self):
        """Pinned host store of the stack's experts: the generated layers, every
        layer key reading the stored layer it repeats (the copies move the bytes
        of 43 distinct layers)."""
        from mixture_experts_gate_amd.layer import HostExperts
        return HostExperts(self.blobs, self.lay, alias=lambda l, e: (l % self.D) * self.cfg.E + e,
                           device=self.dev)

    def logits(self, torch, T, steps):
        """Router logits of every layer for each of the given steps (fresh Gumbel
        noise per step and layer; the Zipf popularity permutation changes every
        256 steps), device tensor [len(steps)][L][T][E]."""
        import numpy as np
        from mixture_experts_gate_amd import synth
        a = np.stack([np.stack([synth.router_logits(self.cfg, T, step=s, layer=l)
                                for l in range(self.L)]) for s in steps])
        return torch.from_numpy(a).to(self.dev)


def run_stack_resident(torch, st, Ts, steps, warmup):
    """All 43 layers resident in HBM; a step is 43 layers, replayed from a graph."""
    from mixture_experts_gate_amd import synth
    from mixture_experts_gate_amd.layer import MoeLayer, expert_table, pack_to_device
    c, lay, dev = st.cfg, st.lay, st.dev
    packed = [pack_to_device(b, lay, dev) for b in st.blobs]
    spacked = [pack_to_device(b[None, :], lay, dev) for b in st.shared_blobs]
    bufs = [packed[l % st.D].clone() for l in range(st.L)]
    sbufs = [spacked[l % st.D].clone() for l in range(st.L)]
    del packed, spacked
    tabs = [expert_table(b.data_ptr(), c.E, lay, device=dev) for b in bufs]
    stabs = [expert_table(b.data_ptr(), 1, lay, device=dev) for b in sbufs]
    out = {}
    for T in Ts:
        # four input steps replayed in turn: two of the first popularity phase,
        # two of the second
        lg = st.logits(torch, T, (0, 1, 256, 257))
        x0 = torch.from_numpy(synth.activations(c, T).view("int16")).to(dev)
        layers = [MoeLayer(c.H, c.E, c.k, c.I, c.fmt, T, shared=True, device=dev) for _ in (0, 1)]
        for ly in layers:
            ly.prepare_shared(T)

        class W:
            def step(self_, i):
                x = x0
                for l in range(st.L):
                    x = layers[l % 2].forward(T, x, tabs[l], logits=lg[i % 4][l],
                                              shared_table=stabs[l])

        ms, wall = time_graphs(torch, W(), steps, warmup)
        ms_step = ms / steps
        # bytes: the distinct experts each layer's router picks, read once
        import numpy as np
        nbytes = 0
        for l in range(st.L):
            layers[0].route(T, logits=lg[0][l], write_logits=False)
            torch.cuda.synchronize()
            u = len(np.unique(layers[0].topk_ids[:T].cpu().numpy()))
            nbytes += (u + 1) * lay.nbytes + 2 * T * c.H * 2
        out[f"T{T}"] = {"T": T, "tokens_per_s": T / (ms_step / 1000.0), "ms_per_step": ms_step,
                        "host_wall_ms_per_step": 1000.0 * wall / steps,
                        "step_algorithmic_bytes": nbytes,
                        "hbm_GBs": nbytes / (ms_step / 1000.0) / 1e9,
                        "hbm_frac": nbytes / (ms_step / 1000.0) / 1e9 / HBM_PEAK_GBS}
        log(f"stack resident T={T}: {out[f'T{T}']['tokens_per_s']:.0f} tok/s, "
            f"{ms_step:.3f} ms/step, HBM {out[f'T{T}']['hbm_frac']*100:.1f}%")
    del bufs, sbufs, tabs, stabs
    torch.cuda.empty_cache()
    return out


def h2d_peak(torch, dev, nbytes=1 << 30):
    """Pinned host -> device copy rate on a side stream (the link reference)."""
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    s = torch.cuda.Stream(dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        a.record(s)
        for _ in range(3):
            dst.copy_(src, non_blocking=True)
        b.record(s)
    torch.cuda.synchronize()
    gbs = 3 * nbytes / (a.elapsed_time(b) / 1000.0) / 1e9
    del src, dst
    return gbs


def run_stack_cached(torch, st, runs, pool_bytes, resize_T=1, resize_steps=32, store=None):
    """The stack through a pool_bytes LRU expert cache fed from pinned host
    memory: per layer, route on the GPU, read the ids back, prefetch the misses
    (hipMemcpyAsync on the copy stream), then the expert FFN, shared expert and
    combine. Shared experts stay resident. runs: [(T, first_step, warmup,
    steps)]: steps first_step .. first_step + steps - 1 are timed after `warmup`
    untimed steps just before them (router logits per step index, Zipf
    popularity re-drawn every 256 steps). After the timed steps at T = resize_T
    the pool is resized to half and back, each followed by resize_steps steps."""
    from mixture_experts_gate_amd import synth
    from mixture_experts_gate_amd.layer import ExpertCache, MoeLayer, expert_table, pack_to_device
    c, lay, dev = st.cfg, st.lay, st.dev
    store = store if store is not None else st.host_store()
    spacked = [pack_to_device(b[None, :], lay, dev) for b in st.shared_blobs]
    stabs = [expert_table(spacked[l % st.D].data_ptr(), 1, lay, device=dev) for l in range(st.L)]
    link = h2d_peak(torch, dev)
    log(f"pinned H2D copy rate: {link:.1f} GB/s")
    out = {"h2d_link_GBs": link, "pool_bytes": pool_bytes}
    for T, first, warmup, steps in runs:
        cache = ExpertCache(store, st.L, c.E, pool_bytes, device=dev)
        extra = 2 * resize_steps if T == resize_T else 0
        s0 = first - warmup
        lg = st.logits(torch, T, range(s0, first + steps + extra))
        x0 = torch.from_numpy(synth.activations(c, T).view("int16")).to(dev)
        layers = [MoeLayer(c.H, c.E, c.k, c.I, c.fmt, T, shared=True, device=dev) for _ in (0, 1)]
        for ly in layers:
            ly.prepare_shared(T)

        def step(i):
            x = x0
            for l in range(st.L):
                ly = layers[l % 2]
                ly.route_permute(T, logits=lg[i - s0][l], write_logits=False)
                ids = ly.topk_ids[:T].cpu().numpy().ravel()
                tab = cache.prefetch(l, ids)
                ly.ffn_combine(T, x, tab, stabs[l])
                x = ly.out[:T]

        for i in range(s0, first):
            step(i)
        torch.cuda.synchronize()
        h0, m0, b0 = cache.stats()
        t0 = time.perf_counter()
        phases = {}
        for i in range(first, first + steps):
            step(i)
            if (i - first) % 64 == 63:
                log(f"stack cached T={T}: step {i}")
            phases.setdefault(i // synth.ZIPF_PHASE_STEPS, 0)
            phases[i // synth.ZIPF_PHASE_STEPS] += 1
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        h1, m1, b1 = cache.stats()
        hits, misses, nb = h1 - h0, m1 - m0, b1 - b0
        r = {"T": T, "steps": steps, "first_step": first, "warmup": warmup,
             "slots": cache.slots(),
             "tokens_per_s": T * steps / el, "ms_per_step": 1000.0 * el / steps,
             "hit_rate": hits / max(hits + misses, 1), "misses_per_step": misses / steps,
             "h2d_bytes_per_step": nb / steps, "h2d_GBs": nb / el / 1e9,
             "h2d_frac_of_link": nb / el / 1e9 / link,
             "popularity_phases": {str(k): v for k, v in sorted(phases.items())}}
        out[f"T{T}"] = r
        log(f"stack cached T={T} steps {first}..{first + steps - 1}: {r['tokens_per_s']:.1f} tok/s, "
            f"hit {r['hit_rate']:.3f}, H2D {r['h2d_GBs']:.1f} GB/s "
            f"({r['h2d_frac_of_link']*100:.0f}% of the copy rate), phases {r['popularity_phases']}")
        if T == resize_T:
            # elastic resize: the pool shrinks to half into a new buffer (the
            # other half could go to other uses), runs, then grows back
            nxt = first + steps
            r["resize"] = []
            for frac in (0.5, 1.0):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                moved = cache.resize(int(pool_bytes * frac))
                torch.cuda.synchronize()
                el = time.perf_counter() - t0
                h0, m0, _ = cache.stats()
                for i in range(nxt, nxt + resize_steps):
                    step(i)
                torch.cuda.synchronize()
                nxt += resize_steps
                h1, m1, _ = cache.stats()
                mb = moved * lay.nbytes
                q = {"pool_bytes": int(pool_bytes * frac), "slots": cache.slots(),
                     "experts_moved": moved, "moved_bytes": mb, "ms": 1000.0 * el,
                     "d2d_GBs_read_plus_write": 2 * mb / el / 1e9,
                     "d2d_hbm_frac": 2 * mb / el / 1e9 / HBM_PEAK_GBS,
                     "hit_rate_next_steps": (h1 - h0) / max(h1 - h0 + m1 - m0, 1),
                     "next_steps": resize_steps}
                r["resize"].append(q)
                log(f"stack cached T={T}: resize to {q['pool_bytes']/1e9:.0f} GB moved {moved} experts "
                    f"({mb/1e9:.1f} GB) in {q['ms']:.1f} ms "
                    f"({q['d2d_hbm_frac']*100:.0f}% of HBM), hit rate over the next "
                    f"{resize_steps} steps {q['hit_rate_next_steps']:.3f}")
        cache.close()
        del cache, lg
    return out


def run_prefill_stream(torch, st, T=4096, n_layers=6, store=None):
    """Full-layer double-buffered prefill streaming over the stack (the pages'
    prefill mechanism): every expert of layer l+1 is requested while layer l
    computes, into a pool of two layers, from pinned host memory. Reported: the
    time per layer streamed, the compute alone (the same layers with their
    experts already in the pool), the copy alone (one layer's experts with no
    compute), the overlap (max(copy, compute) over the streamed time) and the
    H2D rate against the measured pinned copy rate."""
    from mixture_experts_gate_amd import synth
    from mixture_experts_gate_amd.layer import ExpertCache, MoeLayer, expert_table, pack_to_device
    c, lay, dev = st.cfg, st.lay, st.dev
    store = store if store is not None else st.host_store()
    spacked = [pack_to_device(b[None, :], lay, dev) for b in st.shared_blobs]
    stabs = [expert_table(spacked[l % st.D].data_ptr(), 1, lay, device=dev) for l in range(st.L)]
    slot = (lay.nbytes + 255) // 256 * 256
    cache = ExpertCache(store, st.L, c.E, 2 * c.E * slot, device=dev)
    ly = MoeLayer(c.H, c.E, c.k, c.I, c.fmt, T, shared=True, device=dev)
    ly.prepare_shared(T)
    x0 = torch.from_numpy(synth.activations(c, T).view("int16")).to(dev)
    lg = st.logits(torch, T, (0,))[0]
    link = h2d_peak(torch, dev)
    layer_bytes = c.E * lay.nbytes

    def copy_only(l):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        cache.prefetch(l, None)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def streamed(first, n):
        x = x0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        tab = cache.prefetch(first, None)
        for l in range(first, first + n):
            ly.forward(T, x, tab, logits=lg[l], shared_table=stabs[l])
            x = ly.out[:T]
            if l + 1 < first + n:
                tab = cache.prefetch(l + 1, None)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def compute_only(l, reps=5):
        tab = cache.prefetch(l, None)          # resident from the pass before: all hits
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            ly.forward(T, x0, tab, logits=lg[l], shared_table=stabs[l])
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps

    streamed(0, 2)                                # warm-up
    t_copy = copy_only(2)
    t_stream = streamed(3, n_layers)
    t_comp = compute_only(3 + n_layers - 1)
    per = t_stream / n_layers
    h, m, b = cache.stats()
    cache.close()
    r = {"T": T, "layers": n_layers, "layer_bytes": layer_bytes, "h2d_link_GBs": link,
         "ms_per_layer_streamed": 1000.0 * per, "ms_per_layer_compute_only": 1000.0 * t_comp,
         "ms_per_layer_copy_only": 1000.0 * t_copy,
         "overlap_efficiency": max(t_copy, t_comp) / per,
         "h2d_GBs_streamed": layer_bytes / per / 1e9,
         "h2d_frac_of_link": layer_bytes / per / 1e9 / link,
         "tokens_per_s": T / per}
    log(f"prefill streaming T={T}: {r['ms_per_layer_streamed']:.1f} ms/layer streamed, "
        f"copy alone {r['ms_per_layer_copy_only']:.1f} ms, compute alone "
        f"{r['ms_per_layer_compute_only']:.2f} ms, overlap {r['overlap_efficiency']:.2f}, "
        f"H2D {r['h2d_GBs_streamed']:.1f} GB/s ({r['h2d_frac_of_link']*100:.0f}% of the copy rate)")
    return r


def cpu_baseline(wl, budget_s=12.0):
    """Oracle on the same layer, single thread pinned to one core."""
    import oracle
    oracle.build(force=False)
    try:
        cpus = sorted(os.sched_getaffinity(0))
        old = set(cpus)
        os.sched_setaffinity(0, {cpus[-1]})
    except (AttributeError, OSError):
        old = None
    x, lg = wl.x_host[0], wl.lg_host[0]
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.moe_layer(x, wl.lay, wl.pool, wl.cfg.k, logits=lg)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    if old is not None:
        os.sched_setaffinity(0, old)
    return {"value": wl.T * reps / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full layer passes at T={wl.T} (same layer, input batch 0), "
                      f"single-threaded C oracle, fp64 accumulation, {el:.1f} s",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def micro(torch, dev):
    """References measured on this GPU with the library's measurement kernels:
    the read-stream rate at the byte counts of the decode kernels (and larger),
    with a persistent grid (two workgroups per compute unit) and with one
    workgroup per 64 KB chunk, buffers rotated over more than 1 GB so that the
    bytes come from HBM; and the issue rate of the bf16 and the block-scaled
    FP8 x FP4 matrix instructions. Times are the dispatches' own start/end
    events (library timing mode)."""
    from mixture_experts_gate_amd import _lib
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    kid = {n: i for i, n in enumerate(_lib.kernel_names())}
    out = {"read_stream": [], "mfma": [], "compute_units": ncu}

    def timed(fn, reps, name):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        _lib.moe_set_option(_lib.MOE_OPT_TIMING, 1)
        for i in range(reps):
            fn(i)
        torch.cuda.synchronize()
        n, ms = _lib.moe_timing_query(kid[name])
        _lib.moe_set_option(_lib.MOE_OPT_TIMING, 0)
        return 1000.0 * ms / n

    for size in (105_000_000, 211_000_000, 316_000_000, 1_000_000_000, 4_000_000_000):
        nbytes = size // 65536 * 65536
        nbuf = max(2, -(-1_100_000_000 // nbytes))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        for b in bufs:
            b.fill_(1)
        for label, grid in (("persistent", 2 * ncu), ("one_per_chunk", nbytes // 65536)):
            us = timed(lambda i: _lib.moe_micro_read(bufs[i % nbuf], nbytes, grid, sink),
                       4 * nbuf, "micro_read")
            out["read_stream"].append({"bytes": nbytes, "grid": grid, "launch": label, "avg_us": us,
                                       "GBs": nbytes / (us * 1e-6) / 1e9})
            log(f"read stream {nbytes/1e6:.0f} MB, {label} grid {grid}: {us:.1f} us, "
                f"{nbytes/(us*1e-6)/1e9:.0f} GB/s")
        del bufs
    torch.cuda.empty_cache()
    # per-launch floor: back-to-back dependent launches replayed from a graph,
    # each one workgroup reading 64 KB (one round trip to memory), and the
    # same with 256 workgroups reading 16 MB (start-up of a full-chip launch)
    floor = []
    for nbytes, grid in ((65536, 1), (16 << 20, 256)):
        small = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        small.fill_(1)
        n = 32
        _lib.moe_micro_read(small, nbytes, grid, sink)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                _lib.moe_micro_read(small, nbytes, grid, sink)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = 1000.0 * e0.elapsed_time(e1) / (10 * n)
        floor.append({"bytes": nbytes, "grid": grid, "us_per_launch": us})
        log(f"launch floor: {grid} workgroup(s) reading {nbytes/1e6:.2f} MB, {us:.2f} us per launch "
            f"in a graph")
        del g, small
    out["launch_floor"] = floor
    for kind, label in ((0, "bf16_32x32x16"), (1, "scaled_fp4xfp8_16x16x128")):
        grid, iters = 4 * ncu, 2000
        flops = _lib.moe_micro_mfma(kind, grid, iters, sink)
        us = timed(lambda i: _lib.moe_micro_mfma(kind, grid, iters, sink), 5, "micro_mfma")
        out["mfma"].append({"instruction": label, "grid": grid, "avg_us": us,
                            "TFLOPs": flops / (us * 1e-6) / 1e12})
        log(f"matrix cores {label}: {flops/(us*1e-6)/1e12:.0f} TFLOP/s")
    return out


def read_peak_for(micro_res, nbytes):
    """Best measured read-stream rate at the size closest to nbytes."""
    if not micro_res:
        return None
    rs = micro_res["read_stream"]
    size = min({r["bytes"] for r in rs}, key=lambda b: abs(b - nbytes))
    return max(r["GBs"] for r in rs if r["bytes"] == size)


def calibrate_host_expert(torch, dev, store, keys, H, I, threads=0):
    """Host expert kernel cost: seconds per expert (its weights decoded) and per
    token row, from timing calls at 1 and 8 rows over distinct experts' pinned
    blobs in turn (so the weights come from host memory, not the host's
    caches) while host-to-device copies stream on a side stream, as the
    cache's copies do while the host computes its experts."""
    import numpy as np
    from mixture_experts_gate_amd import _lib
    rng = np.random.default_rng(0)
    # copy traffic for the timing window: 512 MB pinned -> device, repeated
    src = torch.empty(512 << 20, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(side):
        for _ in range(48):            # about 0.4 s at the native link
            dst.copy_(src, non_blocking=True)
    t = {}
    for n in (1, 8):
        x = (rng.standard_normal((n, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        y = np.empty_like(x)
        _lib.moe_cpu_expert_ffn(_lib.MOE_W_MXFP4, *store.blob_ptrs(keys[0]), H, I, x, y, threads)
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 0.15:
            _lib.moe_cpu_expert_ffn(_lib.MOE_W_MXFP4, *store.blob_ptrs(keys[reps % len(keys)]), H, I,
                                    x, y, threads)
            reps += 1
        t[n] = (time.perf_counter() - t0) / reps
    side.synchronize()
    del src, dst
    per_row = max((t[8] - t[1]) / 7.0, 0.0)
    return t[1] - per_row, per_row


def calibrate_host_fixed(torch, dev, H):
    """The fixed cost of giving the host any expert in a layer: the rows sent
    back (pinned copy, scatter, synchronisation) and a wake-up of the host
    kernel's threads, measured with a one-row call at the smallest shapes."""
    import numpy as np
    from mixture_experts_gate_amd import _lib
    src = torch.zeros((1, H), dtype=torch.bfloat16, device=dev)
    dst = torch.zeros((8, H), dtype=torch.bfloat16, device=dev)
    idx = torch.zeros(1, dtype=torch.int32, device=dev)
    pin = torch.zeros((1, H), dtype=torch.int16, pin_memory=True)
    blob = np.zeros(128 * 128 * 2, dtype=np.uint8)
    x = np.zeros((1, 128), dtype=np.uint16)
    y = np.empty_like(x)
    p = blob.ctypes.data

    def once():
        _lib.moe_cpu_expert_ffn(_lib.MOE_W_MXFP4, p, p, p, p, 128, 128, x, y, 0)
        src.view(torch.int16).copy_(pin, non_blocking=True)
        _lib.moe_scatter_rows(src, idx, 1, H * 2, dst)
        torch.cuda.synchronize()

    for _ in range(10):
        once()
    t0, reps = time.perf_counter(), 0
    while time.perf_counter() - t0 < 0.2:
        once()
        reps += 1
    return (time.perf_counter() - t0) / reps


def run_qstar(torch, st, store, pool_bytes, T=1, warmup=8, steps=24, links=(None, 14.0, 5.0)):
    """Bandwidth-adaptive placement (q*) on the cached stack: per layer the
    misses are computed on the host CPU from their pinned blobs while that is
    cheaper than copying them at the rate the cache measures, against copying
    every miss (stream only). Links: the native one and slower ones emulated by
    holding the copy stream (the pages' desktop PCIe 4.0 and x8 laptop links
    move the ~140 GB pool in about 5 and over 10 seconds)."""
    from mixture_experts_gate_amd import _lib, synth
    from mixture_experts_gate_amd.layer import ExpertCache, MoeLayer, expert_table, pack_to_device
    c, lay, dev = st.cfg, st.lay, st.dev
    spacked = [pack_to_device(b[None, :], lay, dev) for b in st.shared_blobs]
    stabs = [expert_table(spacked[l % st.D].data_ptr(), 1, lay, device=dev) for l in range(st.L)]
    a, b = calibrate_host_expert(torch, dev, store, list(range(0, 64 * 7, 7)), c.H, c.I)
    f = calibrate_host_fixed(torch, dev, c.H)
    native = h2d_peak(torch, dev)
    crossover = lay.nbytes / (a + b) / 1e9
    log(f"host expert kernel: {a*1e3:.2f} ms per expert + {b*1e3:.3f} ms per row, "
        f"{f*1e3:.3f} ms fixed per layer; a one-row miss is cheaper on the host below "
        f"{crossover:.1f} GB/s (link {native:.1f} GB/s)")
    out = {"host_s_fixed": f, "host_s_per_expert": a, "host_s_per_row": b,
           "crossover_GBs_one_row": crossover,
           "native_link_GBs": native, "expert_bytes": lay.nbytes, "runs": []}
    lg = st.logits(torch, T, range(warmup + steps))
    x0 = torch.from_numpy(synth.activations(c, T).view("int16")).to(dev)
    for link in links:
        thr = 0 if link is None else int(1000.0 / (1.0 / link - 1.0 / native))
        _lib.moe_set_option(_lib.MOE_OPT_CACHE_THROTTLE_MBS, thr)
        try:
            for mode in ("stream", "qstar"):
                cache = ExpertCache(store, st.L, c.E, pool_bytes, device=dev)
                ly = MoeLayer(c.H, c.E, c.k, c.I, c.fmt, T, shared=True, device=dev)
                ly.prepare_shared(T)
                host_experts = [0]

                def step(i):
                    x = x0
                    for l in range(st.L):
                        if mode == "qstar":
                            o, mask = ly.forward_cached_qstar(T, x, cache, l, logits=lg[i][l],
                                                              shared_table=stabs[l],
                                                              host_s_fixed=f,
                                                              host_s_per_expert=a,
                                                              host_s_per_row=b,
                                                              live_host=True)
                            host_experts[0] += int(mask.sum())
                        else:
                            ly.route_permute(T, logits=lg[i][l], write_logits=False)
                            ids = ly.topk_ids[:T].cpu().numpy().ravel()
                            tab = cache.prefetch(l, ids)
                            ysh = ly.ffn_with_shared(T, x, tab, stabs[l])
                            ly.combine(T, y_shared=ysh)
                            o = ly.out[:T]
                        x = o

                for i in range(warmup):
                    step(i)
                torch.cuda.synchronize()
                h0, m0, b0 = cache.stats()
                host_experts[0] = 0
                t0 = time.perf_counter()
                for i in range(warmup, warmup + steps):
                    step(i)
                torch.cuda.synchronize()
                el = time.perf_counter() - t0
                h1, m1, b1 = cache.stats()
                gbs, _ = cache.bandwidth()
                live = cache.host_s_per_expert_live
                cache.close()
                r = {"link": "native" if link is None else f"{link:g} GB/s (emulated)",
                     "mode": mode, "T": T, "steps": steps, "tokens_per_s": T * steps / el,
                     "host_s_per_expert_live": live,
                     "ms_per_step": 1000.0 * el / steps, "measured_link_GBs": gbs,
                     "copied_per_step": (m1 - m0) / steps,
                     "host_experts_per_step": host_experts[0] / steps,
                     "hits_per_step": (h1 - h0) / steps}
                out["runs"].append(r)
                log(f"q* leg, link {r['link']}, {mode}: {r['tokens_per_s']:.1f} tok/s, "
                    f"{r['ms_per_step']:.1f} ms/step, copied {r['copied_per_step']:.1f} and "
                    f"host {r['host_experts_per_step']:.1f} experts per step, measured link "
                    f"{gbs:.1f} GB/s" + (f", host {live*1e3:.2f} ms per expert measured live"
                                         if live else ""))
        finally:
            _lib.moe_set_option(_lib.MOE_OPT_CACHE_THROTTLE_MBS, 0)
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baselines(c2_pool, budget_s=3.0):
    """The oracle on every workload (one core, pinned): full layers where the
    oracle finishes in seconds, token subsets of the large batches with the
    per-token linear extrapolation to the full batch labelled as such (the
    layer is token-independent once routing is fixed), and a sample of layers
    of one 43-layer stack step."""
    import numpy as np
    import oracle
    from mixture_experts_gate_amd import synth
    oracle.build(force=False)
    try:
        cpus = sorted(os.sched_getaffinity(0))
        old = set(cpus)
        os.sched_setaffinity(0, {cpus[-1]})
    except (AttributeError, OSError):
        old = None
    out = []

    def timed(fn, min_reps=1):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if (el >= budget_s and reps >= min_reps) or reps >= 50:
                return el / reps, reps

    def record(name, T_full, tokens, per_pass, reps, note):
        r = {"workload": name, "T": T_full, "tokens_timed": tokens, "passes": reps,
             "s_per_pass": per_pass, "value": tokens / per_pass, "unit": "tokens/s", "cores": 1,
             "kind": "oracle"}
        if tokens < T_full:
            r["extrapolated_full_batch_s"] = per_pass * T_full / tokens
            r["note"] = ("measured on a token subset; full-batch time extrapolated per token "
                         "(linear, the layer being token-independent once routing is fixed)")
        if note:
            r["sample"] = note
        out.append(r)
        log(f"oracle {name}: {r['value']:.2f} tok/s ({reps} passes of {tokens} tokens)")

    c1 = synth.CONFIGS[1]
    lay1 = synth.blob_layout(c1.H, c1.I, c1.fmt)
    pool1, x1, wg1 = synth.expert_pool(c1), synth.activations(c1, 16), synth.gate_weights(c1)
    per, reps = timed(lambda: oracle.moe_layer(x1, lay1, pool1, c1.k, wg=wg1))
    record("tiny layer T=16 (gate computed)", 16, 16, per, reps, None)
    c2 = synth.CONFIGS[2]
    lay2 = synth.blob_layout(c2.H, c2.I, c2.fmt)
    for T in (1, 8, 32, 64):
        x, lg = synth.activations(c2, T), synth.router_logits(c2, T)
        per, reps = timed(lambda: oracle.moe_layer(x, lay2, c2_pool, c2.k, logits=lg))
        record(f"decode layer T={T}", T, T, per, reps, None)
    c3 = synth.CONFIGS[3]
    sub = np.arange(0, 8192, 32)                    # 256 tokens of the prefill batch
    x3 = synth.activations(c3, 8192)[sub]
    lg3 = synth.router_logits(c3, 8192)[sub]
    per, reps = timed(lambda: oracle.moe_layer(x3, lay2, c2_pool, c3.k, logits=lg3))
    record("prefill layer T=8192", 8192, len(sub), per, reps, "every 32nd token of the batch")
    c4 = synth.CONFIGS[4]
    lay4 = synth.blob_layout(c4.H, c4.I, c4.fmt)
    pool4, sh4 = synth.expert_pool(c4), synth.shared_expert(c4)
    for T, n in ((1, 1), (64, 16), (4096, 64)):
        idx = np.arange(0, T, T // n)
        x, lg = synth.activations(c4, T)[idx], synth.router_logits(c4, T)[idx]
        per, reps = timed(lambda: oracle.moe_layer(x, lay4, pool4, c4.k, logits=lg,
                                                   shared_blob=sh4))
        record(f"large sparse layer T={T}", T, len(idx), per, reps,
               None if n == T else f"every {T // n}th token of the batch")
    # one step of the stack at T=1: 8 of its 43 layers (each with its own
    # experts and logits), scaled to the step
    c5 = synth.CONFIGS[5]
    pool5, sh5 = pool4, sh4           # the stack's layers have the large sparse layer's shapes
    x = synth.activations(c5, 1)
    t0 = time.perf_counter()
    for l in range(8):
        lg = synth.router_logits(c5, 1, layer=l)
        r = oracle.moe_layer(x, lay4, pool5, c5.k, logits=lg, shared_blob=sh5)
        x = r["out_bf16"]
    el = (time.perf_counter() - t0) * c5.layers / 8
    out.append({"workload": "43-layer stack, one step at T=1", "T": 1, "value": 1.0 / el,
                "unit": "tokens/s", "cores": 1, "kind": "oracle", "s_per_step": el,
                "note": "8 of the 43 layers timed, the step scaled by 43/8 (layers cost the same)"})
    log(f"oracle stack step T=1: {el:.1f} s per step")
    if old is not None:
        os.sched_setaffinity(0, old)
    return {"cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "runs": out}


def calib_copy(torch, dev):
    n = 512 << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty(n, dtype=torch.uint8, device=dev)
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"calibration copy of {n} bytes done")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from mixture_experts_gate_amd import _lib, synth
    _lib.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.profile:
        args.no_sweep = True
        args.no_cpu = True
    if args.calib_copy:
        calib_copy(torch, dev)
    only = set(args.only.split(",")) if args.only else None
    want = lambda name: only is None or name in only

    c2 = synth.CONFIGS[2]
    sweep = {}
    log(f"headline: decode layer T={args.T}, {args.steps} steps, {args.warmup} warm-up")
    wl, head = run_workload(torch, c2, args.T, args.steps, args.warmup, dev)
    dom, roof = roofline(head, args.T)
    log(f"T={args.T}: {head['tokens_per_s']:.0f} tok/s, {head['ms_per_step']*1000:.1f} us/step, "
        f"layer HBM {head['layer_hbm_frac']*100:.1f}%")
    if not args.no_sweep and want("decode"):
        for T in (1, 8, 32):
            if T == args.T:
                continue
            _, r = run_workload(torch, c2, T, max(args.steps // 2, 32), args.warmup, dev,
                                pool=wl.pool, dexp=wl.dexp)
            sweep[f"decode_T{T}"] = r
            log(f"T={T}: {r['tokens_per_s']:.0f} tok/s, {r['ms_per_step']*1000:.1f} us/step")
    if not args.no_sweep and want("formats"):
        # the decode layer's shapes and routing with NVFP4 and FP8 expert weights
        import dataclasses
        for f in ("nvfp4", "fp8"):
            cf = dataclasses.replace(c2, name=f"decode_{f}", fmt=f, weights="marginal_" + f)
            fw, r = run_workload(torch, cf, args.T, max(args.steps // 2, 32), args.warmup, dev)
            gu = r["kernels"].get("ffn_decode_gate_up", {})
            r["roofline_gate_up"] = {"bound": "hbm", "achieved": gu.get("GBs"),
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": (gu.get("GBs") or 0.0) / HBM_PEAK_GBS}
            sweep[f"decode_{f}_T{args.T}"] = r
            log(f"{f} weights T={args.T}: {r['tokens_per_s']:.0f} tok/s, "
                f"{r['ms_per_step']*1000:.1f} us/step, gate/up {gu.get('GBs', 0):.0f} GB/s "
                f"({r['roofline_gate_up']['frac']*100:.1f}% of HBM), layer HBM "
                f"{r['layer_hbm_frac']*100:.1f}%")
            if f == "fp8":
                # the prefill workload (T=8192, its routing) with the same FP8 weights:
                # the tiled kernels with E4M3 weights
                cp = dataclasses.replace(synth.CONFIGS[3], name="prefill_fp8", fmt=f,
                                         weights="marginal_" + f)
                _, rp = run_workload(torch, cp, 8192, 16, 3, dev, pool=fw.pool, dexp=fw.dexp,
                                     kernel_steps=8)
                rp["mfma_frac_bf16_peak"] = rp["layer_tflops"] / BF16_PEAK_TFLOPS
                sweep["prefill_fp8_T8192"] = rp
                log(f"fp8 weights T=8192: {rp['tokens_per_s']:.0f} tok/s, "
                    f"{rp['layer_tflops']:.1f} TFLOP/s")
            del fw
            torch.cuda.empty_cache()
    if not args.no_sweep and want("prefill"):
        # the prefill workload runs the same layer (same weights) at T=8192
        _, r = run_workload(torch, synth.CONFIGS[3], 8192, 16, 3, dev, pool=wl.pool,
                            dexp=wl.dexp, kernel_steps=8)
        r["mfma_frac_bf16_peak"] = r["layer_tflops"] / BF16_PEAK_TFLOPS
        sweep["prefill_T8192"] = r
        log(f"T=8192: {r['tokens_per_s']:.0f} tok/s, {r['layer_tflops']:.1f} TFLOP/s")
    if not args.no_sweep and want("cfg4"):
        c4 = synth.CONFIGS[4]
        log("config 4: generating 256 experts + shared ...")
        w4 = None
        c4_T = {int(v) for v in args.cfg4_T.split(",") if v}
        for T, steps in ((1, 100), (2, 100), (64, 100), (4096, 8)):
            if T not in c4_T:
                continue
            # decode sizes rotate 8 weight replicas (27 GB) so that a hot
            # expert's bytes come back from HBM, not from the last-level cache
            w, r = run_workload(torch, c4, T, steps, 3, dev, replicas=8 if T <= 64 else 2,
                                pool=None if w4 is None else w4.pool,
                                dexp=None if w4 is None else w4.dexp,
                                shared=None if w4 is None else w4.sh,
                                kernel_steps=min(steps, 16))
            w4 = w4 or w
            if T <= 64:
                # the same steps with the shared expert as its own call on a
                # side stream, for the gain of running it in the routed launches
                w.fuse_shared = False
                ms, _ = time_graphs(torch, w, steps, 3)
                w.fuse_shared = True
                r["unfused_shared_ms_per_step"] = ms / steps
            if T == 4096:
                r["mfma_frac_bf16_peak"] = r["layer_tflops"] / BF16_PEAK_TFLOPS
            sweep[f"cfg4_T{T}"] = r
            log(f"config 4 T={T}: {r['tokens_per_s']:.0f} tok/s, {r['ms_per_step']*1000:.1f} us/step, "
                f"layer HBM {r['layer_hbm_frac']*100:.1f}%, {r['layer_tflops']:.1f} TFLOP/s"
                + (f", shared expert as its own call {r['unfused_shared_ms_per_step']*1000:.1f} us/step"
                   if "unfused_shared_ms_per_step" in r else ""))
        del w4
        torch.cuda.empty_cache()
    if not args.no_sweep and not args.no_stack and (want("stack") or want("stream") or
                                                    want("qstar")):
        c5 = synth.CONFIGS[5]
        log("config 5: generating 2 distinct layers ...")
        st = Stack(torch, c5, dev, distinct=2)
        if want("stack"):
            sweep["stack43_resident"] = run_stack_resident(torch, st, (1, 2, 4, 8, 16), 40, 3)
        store = st.host_store()
        if want("stream"):
            sweep["prefill_stream_T4096"] = run_prefill_stream(torch, st, store=store)
        if want("stack"):
            # T=1 over four popularity phases; T=16 across the change at step 256
            runs = [(1, 32, 32, args.stack_steps), (2, 128, 4, 16), (4, 128, 4, 16),
                    (8, 128, 4, 16), (16, 248, 4, 16)]
            sweep["stack43_cache32GB"] = run_stack_cached(torch, st, runs, 32 * 10**9,
                                                          store=store)
        if want("qstar"):
            sweep["stack43_qstar"] = run_qstar(torch, st, store, 32 * 10**9)
        del st, store
    micro_res = None
    if not args.no_micro and not args.profile:
        log("reference measurements: read stream, matrix cores")
        micro_res = micro(torch, dev)
        if roof.get("achieved"):
            peak = read_peak_for(micro_res, roof["algorithmic_bytes_per_launch"])
            roof["measured_read_stream_GBs"] = peak
            roof["frac_of_measured_read_stream"] = roof["achieved"] / peak
    cpu = cpu_all = None
    if not args.no_cpu:
        log("CPU oracle baseline ...")
        cpu = cpu_baseline(wl)
        if not args.no_sweep:
            cpu_all = cpu_baselines(wl.pool)
    c = wl.cfg
    line = {
        "metric": "MoE-layer tokens/s at decode T=1..64 & prefill T=8192; % HBM / MFMA roofline",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "warm_replay_steps": head["warm_replay_steps"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode-shaped routed MoE layer H={c.H} E={c.E} top-{c.k} "
                               f"I={c.I}, MXFP4 expert weights, bf16 activations, T={args.T}",
                   "T": args.T, "H": c.H, "E": c.E, "k": c.k, "I": c.I,
                   "weights": "MXFP4 (E2M1 + E8M0 per 32 along K)", "weight_replicas": REPLICAS,
                   "unique_experts_per_step": head["unique_experts"],
                   "layer_hbm_frac": head["layer_hbm_frac"],
                   "layer_hbm_GBs": head["layer_hbm_GBs"],
                   "kernels": head["kernels"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "cpu_baseline_sweep": cpu_all,
        "micro": micro_res,
        "sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
