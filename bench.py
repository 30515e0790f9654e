#!/usr/bin/env python3
"""MoE-layer throughput on one MI355X.

One step = one pass of the routed MoE expert layer (route -> permute ->
grouped SwiGLU expert FFN -> combine) over one batch of synthetic tokens, all
inputs resident in HBM. The headline workload is the decode-shaped layer
(H=2048, 128 experts, top-8, I=768, MXFP4 weights, bf16 activations, uniform
router logits) at T=64 tokens; the JSON line also carries T=1, 8, 32 and the
prefill-shaped T=8192 batch of the same layer.

Timing: W eager warm-up steps, then K steps replayed from HIP graphs (one
graph holds 16 consecutive steps), bracketed by device synchronisation.
Steps rotate over 8 replicas of the expert weights (8 x 321 MB, well above the
256 MB last-level cache) and 8 input batches, so weight bytes come from HBM.

roofline: the dominant kernel's algorithmic bytes per launch divided by its
average launch time, from events the library records around each of its
launches on the launch stream (a second pass of K eager steps).
cpu_baseline: the CPU oracle (single-threaded C, fp64) on the same layer.
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
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 512 MiB device copy (HBM counter calibration)")
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
    def __init__(self, torch, T, dev, replicas=REPLICAS, pool=None, dexp=None):
        from mixture_experts_gate_amd import synth
        from mixture_experts_gate_amd.layer import DeviceExperts, MoeLayer
        self.cfg = synth.CONFIGS[2] if T <= 64 else synth.CONFIGS[3]
        c = self.cfg
        self.T = T
        self.lay = synth.blob_layout(c.H, c.I, c.fmt)
        self.pool = synth.expert_pool(c) if pool is None else pool
        self.dexp = DeviceExperts(self.pool, self.lay, copies=replicas, device=dev) if dexp is None else dexp
        self.R = len(self.dexp.tables)
        to16 = lambda a: torch.from_numpy(a.view("int16")).to(dev)
        self.x_host = [synth.activations(c, T, step=r) for r in range(self.R)]
        self.lg_host = [synth.router_logits(c, T, step=r) for r in range(self.R)]
        self.x = [to16(a) for a in self.x_host]
        self.lg = [torch.from_numpy(a).to(dev) for a in self.lg_host]
        self.layer = MoeLayer(c.H, c.E, c.k, c.I, c.fmt, T, device=dev)

    def step(self, i):
        r = i % self.R
        self.layer.forward(self.T, self.x[r], self.dexp.tables[r], logits=self.lg[r])

    def unique_experts(self):
        """Distinct experts touched per step (average over the input batches)."""
        import numpy as np
        import oracle  # only for the host-side count of routed experts
        us = []
        for lg in self.lg_host:
            ids, _, _ = oracle.topk(lg, self.cfg.k)
            us.append(len(np.unique(ids)))
        return float(np.mean(us)), us


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
    # warm replay
    graphs[0][0].replay()
    torch.cuda.synchronize()
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
    from mixture_experts_gate_amd import _lib
    _lib.moe_set_option(_lib.MOE_OPT_TIMING, 1)
    for i in range(steps):
        wl.step(i)
    torch.cuda.synchronize()
    rep = _lib.timing_report()
    _lib.moe_set_option(_lib.MOE_OPT_TIMING, 0)
    return {k: {"launches": n, "avg_us": 1000.0 * ms / n} for k, (n, ms) in rep.items()}


def algorithmic_bytes(wl, U):
    """Bytes each kernel must move at minimum (weights of touched experts read
    once, activations read once, outputs written once)."""
    c, T, lay = wl.cfg, wl.T, wl.lay
    H, I, E, k = c.H, c.I, c.E, c.k
    w13 = lay.w2 - lay.w13           # W13 codes + scales of one expert
    w2 = lay.nbytes - lay.w2         # W2 codes + scales
    n = T * k
    return {
        "route": T * E * 4 + n * 8,
        "permute_small": n * 4 + n * 8 + (E + 1) * 4,
        "ffn_decode_gate_up": U * w13 + T * H * 2 + n * I * 2,
        "ffn_decode_down": U * w2 + n * I * 2 + n * H * 2,
        "ffn_prefill_gate_up": U * w13 + T * H * 2 + n * I * 2,
        "ffn_prefill_down": U * w2 + n * I * 2 + n * H * 2,
        "combine": n * H * 2 + n * 4 + T * H * 2,
        "layer": U * lay.nbytes + 2 * T * H * 2 + T * E * 4 + n * 8,
    }


def run_workload(torch, T, steps, warmup, dev, pool=None, dexp=None, kernel_steps=None):
    wl = Workload(torch, T, dev, pool=pool, dexp=dexp)
    U, _ = wl.unique_experts()
    ms, wall = time_graphs(torch, wl, steps, warmup)
    kt = kernel_timing(torch, wl, kernel_steps or min(steps, 64))
    ab = algorithmic_bytes(wl, U)
    ms_step = ms / steps
    c = wl.cfg
    flops = 6.0 * c.H * c.I * T * c.k
    res = {
        "T": T,
        "tokens_per_s": T * steps / (ms / 1000.0),
        "ms_per_step": ms_step,
        "host_wall_ms_per_step": 1000.0 * wall / steps,
        "unique_experts": U,
        "layer_algorithmic_bytes": ab["layer"],
        "layer_hbm_GBs": ab["layer"] / (ms_step / 1000.0) / 1e9,
        "layer_hbm_frac": ab["layer"] / (ms_step / 1000.0) / 1e9 / HBM_PEAK_GBS,
        "layer_tflops": flops / (ms_step / 1000.0) / 1e12,
        "kernels": kt,
    }
    for name, v in kt.items():
        if name in ab:
            v["algorithmic_bytes"] = ab[name]
            v["GBs"] = ab[name] / (v["avg_us"] * 1e-6) / 1e9
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
                 "timing": "library events around each launch, K eager steps"}


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
            "host_cpus": os.cpu_count()}


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
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from mixture_experts_gate_amd import _lib
    _lib.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.profile:
        args.no_sweep = True
        args.no_cpu = True
    if args.calib_copy:
        calib_copy(torch, dev)

    log(f"headline: decode layer T={args.T}, {args.steps} steps, {args.warmup} warm-up")
    wl, head = run_workload(torch, args.T, args.steps, args.warmup, dev)
    dom, roof = roofline(head, args.T)
    log(f"T={args.T}: {head['tokens_per_s']:.0f} tok/s, {head['ms_per_step']*1000:.1f} us/step, "
        f"layer HBM {head['layer_hbm_frac']*100:.1f}%")
    sweep = {}
    if not args.no_sweep:
        for T in (1, 8, 32):
            if T == args.T:
                continue
            _, r = run_workload(torch, T, max(args.steps // 2, 32), args.warmup, dev,
                                pool=wl.pool, dexp=wl.dexp)
            sweep[f"decode_T{T}"] = r
            log(f"T={T}: {r['tokens_per_s']:.0f} tok/s, {r['ms_per_step']*1000:.1f} us/step")
        _, r = run_workload(torch, 8192, 16, 3, dev, pool=wl.pool, dexp=wl.dexp, kernel_steps=8)
        r["mfma_frac_bf16_peak"] = r["layer_tflops"] / BF16_PEAK_TFLOPS
        sweep["prefill_T8192"] = r
        log(f"T=8192: {r['tokens_per_s']:.0f} tok/s, {r['layer_tflops']:.1f} TFLOP/s")
    cpu = None
    if not args.no_cpu:
        log("CPU oracle baseline ...")
        cpu = cpu_baseline(wl)
    c = wl.cfg
    line = {
        "metric": "MoE-layer tokens/s at decode T=1..64 & prefill T=8192; % HBM / MFMA roofline",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
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
        "sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
