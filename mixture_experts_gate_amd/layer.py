"""Device-side orchestration of one MoE layer on top of the C ABI.

PyTorch only provides device memory and the stream; every step of the layer
(routing, permutation, expert FFN, combine, cache copies) is a call into
``libmoe.so``. Buffers are allocated once per (layer shape, max T) and reused.
"""
from __future__ import annotations

import time

import numpy as np
import torch

from . import _lib
from .synth import blob_layout

# moe_permute_ffn_combine derives the permutation in its gate/up launch from
# 8 up to 512 pairs (more make it the two calls, which the layer then makes).
# Below 8 pairs (config 4 at one token: 6 pairs over 256 experts, 33.2
# against 32.8 us per step) the one-launch router + permutation of
# moe_route_permute costs less; from 8 pairs the router alone and the
# permutation in the gate/up launch win (config 2, T=1..8: 0.7 to 1.0 us,
# T=9..64: 3.2 to 3.8 us per step).
_PERMUTE_IN_FFN_PAIRS = (8, 512)
# activation rows (T*k, + T with the shared expert) up to which forward()
# tries the one-launch layer (moe_layer_fused) when the logits are given
_ONE_LAUNCH_ROWS = 31

FMT = {"bf16": _lib.MOE_W_BF16, "mxfp4": _lib.MOE_W_MXFP4, "nvfp4": _lib.MOE_W_NVFP4,
       "fp8": _lib.MOE_W_FP8}


def expert_table(base_ptr: int, n: int, layout, stride: int | None = None, device="cuda"):
    """Device array [n] of moe_expert_w for n blobs laid out every `stride` bytes."""
    stride = layout.nbytes if stride is None else stride
    offs = np.array([layout.w13, layout.s13, layout.w2, layout.s2], dtype=np.int64)
    if layout.fmt == "bf16":
        offs[1] = offs[3] = 0
    tab = (base_ptr + np.arange(n, dtype=np.int64)[:, None] * stride + offs[None, :])
    if layout.fmt == "bf16":
        tab[:, 1] = 0
        tab[:, 3] = 0
    return torch.from_numpy(np.ascontiguousarray(tab)).to(device)


def pack_to_device(pool: np.ndarray, layout, device="cuda"):
    """Upload expert blobs [n][nbytes] in the interchange layout and return a
    device tensor of the same shape in the kernel layout (MXFP4, NVFP4 and FP8
    blocks packed by the library; bf16 blobs are used as they are)."""
    host = torch.from_numpy(np.ascontiguousarray(pool, dtype=np.uint8))
    if host.dim() == 1:
        host = host[None, :]
    src = host.to(device)
    if layout.fmt == "bf16":
        return src
    dst = torch.empty_like(src)
    n, nb = src.shape
    _lib.moe_pack_weights(FMT[layout.fmt], src, dst, n, nb, nb, layout.H, layout.I, layout)
    torch.cuda.synchronize()
    del src
    return dst


class DeviceExperts:
    """Expert blobs resident in HBM in the kernel layout (``copies`` identical
    replicas, so that a benchmark can rotate between them and read every byte
    from HBM), plus one moe_expert_w table per replica."""

    def __init__(self, pool: np.ndarray, layout, copies: int = 1, device="cuda"):
        self.layout = layout
        first = pack_to_device(pool, layout, device)
        self.E = first.shape[0]
        self.bufs = [first]
        for _ in range(copies - 1):
            self.bufs.append(first.clone())
        self.tables = [expert_table(b.data_ptr(), self.E, layout, device=device) for b in self.bufs]

    @property
    def table(self):
        return self.tables[0]


class MoeLayer:
    """Buffers and call sequence for one layer shape with at most T_max tokens."""

    def __init__(self, H, E, k, I, fmt, T_max, shared=False, y_fp32=False, device="cuda"):
        self.H, self.E, self.k, self.I = H, E, k, I
        self.fmt = FMT[fmt] if isinstance(fmt, str) else fmt
        self.T_max = T_max
        self.y_fp32 = bool(y_fp32)
        self.shared = shared
        dev = device
        n = T_max * k
        ydt = torch.float32 if y_fp32 else torch.bfloat16
        self.topk_ids = torch.empty((T_max, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T_max, k), dtype=torch.float32, device=dev)
        self.logits = torch.empty((T_max, E), dtype=torch.float32, device=dev)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        self.sorted_pair = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
        self.pair_row = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
        # with a shared expert the weight-streaming kernels keep its T rows of
        # activation after the routed ones, and y holds its T output rows
        pb, _ = _lib.moe_workspace_size(T_max, k, H, I, E)
        _, fb = _lib.moe_workspace_size(T_max, k + 1 if shared else k, H, I, E)
        self.ws_perm_bytes = max(pb, 256)
        self.ws_ffn_bytes = fb
        self.ws_perm = torch.empty(self.ws_perm_bytes, dtype=torch.uint8, device=dev)
        self.ws_ffn = torch.empty(fb, dtype=torch.uint8, device=dev)
        self.y = torch.empty((max(n + (T_max if shared else 0), 1), H), dtype=ydt, device=dev)
        self.out = torch.empty((T_max, H), dtype=torch.bfloat16, device=dev)
        if shared:
            self.sh_pair = torch.arange(T_max, dtype=torch.int32, device=dev)
            self.sh_off = torch.empty(2, dtype=torch.int32, device=dev)
            _, fbs = _lib.moe_workspace_size(T_max, 1, H, I, 1)
            self.ws_sh_bytes = fbs
            self.ws_sh = torch.empty(fbs, dtype=torch.uint8, device=dev)
            self.y_sh = torch.empty((T_max, H), dtype=ydt, device=dev)
        # barrier counters of the one-launch layer (zero before its first call)
        self.sync = torch.zeros(_lib.LAYER_SYNC_BYTES // 8, dtype=torch.int64, device=dev)
        self._sh_T = -1
        self._side = None       # stream of the shared expert (default priority)

    # individual stages ----------------------------------------------------
    def route(self, T, x=None, wg=None, logits=None, renormalize=True, stream=None,
              write_logits=True):
        _lib.moe_route(x, wg, logits, self.logits if write_logits else None, T, self.H, self.E,
                       self.k, renormalize, self.topk_ids, self.topk_w, stream)

    def route_permute(self, T, x=None, wg=None, logits=None, renormalize=True, stream=None,
                      write_logits=True):
        _lib.moe_route_permute(x, wg, logits, self.logits if write_logits else None, T, self.H,
                               self.E, self.k, renormalize, self.topk_ids, self.topk_w,
                               self.offsets, self.sorted_pair, self.pair_row, self.ws_perm,
                               self.ws_perm_bytes, stream)

    def permute(self, T, stream=None):
        _lib.moe_permute(self.topk_ids, T, self.k, self.E, self.offsets, self.sorted_pair,
                         self.pair_row, self.ws_perm, self.ws_perm_bytes, stream)

    def ffn(self, T, x, table, stream=None, perm=None):
        """perm: (sorted_pair, offsets) to use instead of the layer's own."""
        sp, off = perm if perm is not None else (self.sorted_pair, self.offsets)
        _lib.moe_expert_ffn(x, sp, off, table, self.fmt, T, self.k, self.H, self.I, self.E, self.y,
                            self.y_fp32, self.ws_ffn, self.ws_ffn_bytes, stream)

    def combine(self, T, with_shared=False, stream=None, y_shared=None):
        """y_shared: the shared expert's rows (from ffn_with_shared); with_shared
        alone takes them from the separate shared-expert buffer."""
        if y_shared is None and with_shared:
            y_shared = self.y_sh
        _lib.moe_combine(self.y, self.y_fp32, self.topk_w, y_shared, T, self.k, self.H, self.out,
                         stream)

    # whole layer -----------------------------------------------------------
    def forward(self, T, x, table, logits=None, wg=None, shared_table=None, renormalize=True,
                stream=None, write_logits=False, fused_routing=True, fuse_shared=True,
                fuse_combine=True):
        """route -> permute -> expert FFN (+ shared expert) -> combine; returns out[:T].
        fused_routing: route and permute with the one-call entry (one kernel for
        small batches) instead of the two separate calls; from 8 to 512 pairs
        (with fuse_combine, bf16 y) the router, then moe_permute_ffn_combine,
        whose gate/up launch derives the permutation itself.
        fuse_shared: run the shared expert in the routed FFN's launches
        (moe_expert_ffn_shared); else it is its own call on a side stream.
        fuse_combine: the FFN and the combine through moe_expert_ffn_combine
        (one down + combine launch at a handful of tokens; bf16 y only)."""
        if T > self.T_max:
            raise ValueError("T exceeds the buffers' T_max")
        wl = write_logits or logits is None
        if (fused_routing and fuse_combine and fuse_shared and not wl and not self.y_fp32
                and T * (self.k + (shared_table is not None)) <= _ONE_LAUNCH_ROWS):
            # router, permutation, expert FFN and combine in one launch
            rc = _lib.moe_layer_fused(
                x, logits, table, shared_table, self.fmt, T, self.k, self.H, self.I, self.E,
                renormalize, self.topk_ids, self.topk_w, self.offsets, self.sorted_pair,
                self.pair_row, self.y, self.out, self.ws_ffn, self.ws_ffn_bytes, self.sync,
                stream, check=False)
            if rc != _lib.MOE_EUNSUPPORTED:
                return self.out[:T]
        if (fused_routing and fuse_combine and not self.y_fp32
                and (shared_table is None or fuse_shared)
                and _PERMUTE_IN_FFN_PAIRS[0] <= T * self.k <= _PERMUTE_IN_FFN_PAIRS[1]):
            # the router, then the permutation inside the gate/up launch
            self.route(T, x=x, wg=wg, logits=logits, renormalize=renormalize, stream=stream,
                       write_logits=wl)
            _lib.moe_permute_ffn_combine(
                x, self.topk_ids, self.topk_w, table, shared_table, self.fmt, T, self.k, self.H,
                self.I, self.E, self.offsets, self.sorted_pair, self.pair_row, self.y, self.out,
                self.ws_ffn, self.ws_ffn_bytes, stream)
            return self.out[:T]
        if fused_routing:
            self.route_permute(T, x=x, wg=wg, logits=logits, renormalize=renormalize,
                               stream=stream, write_logits=wl)
        else:
            self.route(T, x=x, wg=wg, logits=logits, renormalize=renormalize, stream=stream,
                       write_logits=wl)
            self.permute(T, stream)
        if fuse_combine and not self.y_fp32 and (shared_table is None or fuse_shared):
            if self.ffn_combine(T, x, table, shared_table, stream) is not None:
                return self.out[:T]
        if shared_table is None:
            self.ffn(T, x, table, stream)
            self.combine(T, stream=stream)
            return self.out[:T]
        ysh = self.ffn_with_shared(T, x, table, shared_table, stream, fuse=fuse_shared)
        self.combine(T, stream=stream, y_shared=ysh)
        return self.out[:T]

    def ffn_combine(self, T, x, table, shared_table=None, stream=None):
        """The expert FFN (with the shared expert when shared_table is given)
        and the combine through moe_expert_ffn_combine (bf16 y); returns
        out[:T], or None when the call declines (MOE_EUNSUPPORTED)."""
        rc = _lib.moe_expert_ffn_combine(
            x, self.sorted_pair, self.offsets, table, shared_table, self.fmt, T, self.k, self.H,
            self.I, self.E, self.topk_w, self.y, self.out, self.ws_ffn, self.ws_ffn_bytes, stream,
            check=False)
        return None if rc == _lib.MOE_EUNSUPPORTED else self.out[:T]

    def ffn_with_shared(self, T, x, table, shared_table, stream=None, fuse=True, perm=None):
        """Routed and shared expert FFN; returns the shared expert's output rows
        [T][H] for the combine. With fuse, where the weight-streaming kernels
        run, the shared expert is one more expert of the routed launches (its
        rows land in y after the routed pairs); otherwise it is its own call on
        a side stream, forked before the routed FFN and joined after it."""
        if not self.shared:
            raise ValueError("layer was built without shared-expert buffers")
        n = T * self.k
        sp, off = perm if perm is not None else (self.sorted_pair, self.offsets)
        if fuse:
            rc = _lib.moe_expert_ffn_shared(x, sp, off, table, shared_table,
                                            self.fmt, T, self.k, self.H, self.I, self.E, self.y,
                                            self.y_fp32, self.ws_ffn, self.ws_ffn_bytes, stream,
                                            check=False)
            if rc != _lib.MOE_EUNSUPPORTED:
                return self.y[n:n + T]
        if self._sh_T != T:
            self.prepare_shared(T)
        main = stream if stream is not None else torch.cuda.current_stream()
        if self._side is None:
            self._side = torch.cuda.Stream(device=main.device)
            self._fork = torch.cuda.Event()
            self._join = torch.cuda.Event()
        self._fork.record(main)
        self._side.wait_event(self._fork)
        self.shared_ffn(T, x, shared_table, self._side)
        self._join.record(self._side)
        self.ffn(T, x, table, stream, perm=perm)
        main.wait_event(self._join)
        return self.y_sh[:T]

    def forward_cached_qstar(self, T, x, cache, layer, logits=None, wg=None, shared_table=None,
                             host_s_fixed=0.0, host_s_per_expert=0.0, host_s_per_row=0.0,
                             link_gbs=0.0, threads=0, stream=None, live_host=False):
        """One layer through an expert cache with the bandwidth-adaptive choice
        of the side that computes each missing expert: route and permute on the
        device and read the permutation back; request the experts (a miss goes
        to the host while the host's time stays within the copy time it saves,
        expert_cache_prefetch_qstar); the device FFN over the permutation
        without the host experts (moe_permute_split); the host experts' rows on
        the host CPU from their pinned blobs (moe_cpu_expert_ffn) while the
        device works, copied into y (moe_scatter_rows); then the combine.
        With live_host, the host's cost per expert is the one its expert calls
        have actually taken in earlier layers through this cache (an
        exponentially weighted mean, weight 1/4 for the newest layer, seeded
        by host_s_per_expert), as the link's rate is the one its copies took.
        Returns (out[:T], host_mask). Requires bf16 y and MXFP4 experts."""
        if self.y_fp32 or self.fmt != _lib.MOE_W_MXFP4:
            raise ValueError("the host expert path needs bf16 y and MXFP4 experts")
        main = stream if stream is not None else torch.cuda.current_stream()
        self.route_permute(T, x=x, wg=wg, logits=logits, stream=main, write_logits=logits is None)
        n = T * self.k
        # read back (one synchronisation) before the request below makes the
        # stream wait for copies
        if not hasattr(self, "_rb_off"):
            self._rb_off = torch.empty(self.E + 1, dtype=torch.int32, pin_memory=True)
            self._rb_sp = torch.empty(max(self.T_max * self.k, 1), dtype=torch.int32,
                                      pin_memory=True)
            self._rb_x = torch.empty((self.T_max, self.H), dtype=torch.int16, pin_memory=True)
        with torch.cuda.stream(main):
            self._rb_off.copy_(self.offsets, non_blocking=True)
            self._rb_sp[:n].copy_(self.sorted_pair[:n], non_blocking=True)
            self._rb_x[:T].copy_(x[:T].view(torch.int16), non_blocking=True)
        main.synchronize()
        off = self._rb_off.numpy().copy()
        sp = self._rb_sp[:n].numpy().copy()
        x_host = self._rb_x[:T].numpy().view(np.uint16).copy()
        cnt = np.diff(off)
        ids = np.nonzero(cnt)[0].astype(np.int32)
        if live_host and cache.host_s_per_expert_live is not None:
            host_s_per_expert = cache.host_s_per_expert_live
        tab, mask = _lib.expert_cache_prefetch_qstar(cache.handle, layer, ids, cnt[ids],
                                                     host_s_fixed, host_s_per_expert,
                                                     host_s_per_row, self.E, link_gbs, main)
        d_off, d_sp, h_pairs = _lib.moe_permute_split(off, sp, mask)
        perm = None
        if len(h_pairs):
            if not hasattr(self, "_q_off"):
                nn = max(self.T_max * self.k, 1)
                dev = self.y.device
                self._q_off = torch.empty(self.E + 1, dtype=torch.int32, device=dev)
                self._q_sp = torch.empty(nn, dtype=torch.int32, device=dev)
                self._q_idx = torch.empty(nn, dtype=torch.int32, device=dev)
                self._q_rows = torch.empty((nn, self.H), dtype=torch.bfloat16, device=dev)
                self._q_host = torch.empty((nn, self.H), dtype=torch.int16, pin_memory=True)
                # pinned staging of [offsets | sorted pairs | host pairs]
                self._q_stage = torch.empty(self.E + 1 + 2 * nn, dtype=torch.int32,
                                            pin_memory=True)
            # (the read-backs above waited for this layer's earlier copies, so
            # the pinned buffers are free to refill)
            st = self._q_stage.numpy()
            E1, nd, nh = self.E + 1, len(d_sp), len(h_pairs)
            st[:E1] = d_off
            st[E1:E1 + nd] = d_sp
            st[E1 + nd:E1 + nd + nh] = h_pairs
            with torch.cuda.stream(main):
                self._q_off.copy_(self._q_stage[:E1], non_blocking=True)
                if nd:
                    self._q_sp[:nd].copy_(self._q_stage[E1:E1 + nd], non_blocking=True)
                self._q_idx[:nh].copy_(self._q_stage[E1 + nd:E1 + nd + nh], non_blocking=True)
            perm = (self._q_sp, self._q_off)
        if shared_table is not None:
            ysh = self.ffn_with_shared(T, x, tab, shared_table, main, perm=perm)
        else:
            ysh = None
            self.ffn(T, x, tab, main, perm=perm)
        if len(h_pairs):
            # the host experts, while the device runs its share
            hy = self._q_host[:len(h_pairs)].numpy().view(np.uint16)
            row = 0
            t_host = time.perf_counter()
            for e in np.nonzero(mask)[0]:
                pairs = sp[off[e]:off[e + 1]]
                xr = np.ascontiguousarray(x_host[pairs // self.k])
                yr = np.empty_like(xr)
                _lib.moe_cpu_expert_ffn(self.fmt, *cache.store.blob_ptrs(cache.key_source(layer, e)),
                                        self.H, self.I, xr, yr, threads)
                hy[row:row + len(pairs)] = yr
                row += len(pairs)
            if live_host:
                # this layer's host cost per expert, its rows' share taken out
                n_he = int(mask.sum())
                per = max(time.perf_counter() - t_host - row * host_s_per_row, 0.0) / n_he
                prev = cache.host_s_per_expert_live
                cache.host_s_per_expert_live = per if prev is None else 0.75 * prev + 0.25 * per
            with torch.cuda.stream(main):
                self._q_rows[:len(h_pairs)].view(torch.int16).copy_(self._q_host[:len(h_pairs)],
                                                                    non_blocking=True)
            _lib.moe_scatter_rows(self._q_rows, self._q_idx, len(h_pairs), self.H * 2, self.y, main)
        self.combine(T, stream=main, y_shared=ysh)
        return self.out[:T], mask

    def prepare_shared(self, T):
        """Write the shared expert's offsets {0, T} (outside any timed or captured region)."""
        self.sh_off.copy_(torch.tensor([0, T], dtype=torch.int32))
        torch.cuda.synchronize()
        self._sh_T = T

    def shared_ffn(self, T, x, shared_table, stream=None):
        _lib.moe_expert_ffn(x, self.sh_pair, self.sh_off, shared_table, self.fmt, T, 1, self.H,
                            self.I, 1, self.y_sh, self.y_fp32, self.ws_sh, self.ws_sh_bytes,
                            stream)


def layout_for(cfg):
    return blob_layout(cfg.H, cfg.I, cfg.fmt)


class HostExperts:
    """Expert blobs of several layers in pinned host memory, in the kernel
    layout (packed on the device by the library, then copied back), as the
    source store of an expert cache. ``blobs[l]`` is [E][nbytes] in the
    interchange layout. Keys (layer, expert) may share storage through
    ``alias``: key (l, e) reads stored blob alias(l, e) (a benchmark can then
    stream a stack larger than it stores; the copies move the same bytes)."""

    def __init__(self, blobs, layout, alias=None, device="cuda"):
        self.layout = layout
        self.n_stored = sum(int(b.shape[0]) for b in blobs)
        self.E = int(blobs[0].shape[0])
        nb = layout.nbytes
        self.host = torch.empty((self.n_stored, nb), dtype=torch.uint8, pin_memory=True)
        row = 0
        for b in blobs:
            packed = pack_to_device(b, layout, device)
            self.host[row:row + packed.shape[0]].copy_(packed)
            row += packed.shape[0]
            del packed
        torch.cuda.synchronize()
        self.alias = alias

    def address(self, stored: int) -> int:
        return self.host.data_ptr() + stored * self.layout.nbytes

    def blob_ptrs(self, stored: int):
        """Host addresses (w13, s13, w2, s2) of a stored blob."""
        b, lay = int(self.address(int(stored))), self.layout
        return b + lay.w13, b + lay.s13, b + lay.w2, b + lay.s2

    def sources(self, n_layers: int, n_experts: int):
        """Host address of each key's blob, [n_layers * n_experts]."""
        out = []
        for l in range(n_layers):
            for e in range(n_experts):
                s = l * n_experts + e if self.alias is None else self.alias(l, e)
                out.append(self.address(s))
        return out


class ExpertCache:
    """Owner of a device slot pool and a ``moe_cache`` over it.

    Use: ``tab = cache.prefetch(l, ids)`` and enqueue the compute that reads
    ``tab`` before the next ``prefetch`` call (that call may refill slots handed
    out by the call before this one once their compute is done); the copies of
    a prefetch overlap whatever the compute stream is still running."""

    def __init__(self, store: HostExperts, n_layers: int, n_experts: int, pool_bytes: int,
                 device="cuda", copy_stream=None):
        lay = store.layout
        slot = (lay.nbytes + 255) // 256 * 256
        self.pool = torch.empty(pool_bytes // slot * slot, dtype=torch.uint8, device=device)
        self.slot_bytes = slot
        self.copy_stream = copy_stream if copy_stream is not None else torch.cuda.Stream(device)
        self.store = store
        self.n_experts = n_experts
        self.srcs = store.sources(n_layers, n_experts)
        self.handle = _lib.expert_cache_reserve(self.pool, self.pool.numel(), lay.nbytes, n_layers,
                                                n_experts, self.srcs, lay,
                                                self.copy_stream.cuda_stream)
        # host cost per expert measured by the q* path (forward_cached_qstar)
        self.host_s_per_expert_live = None

    def prefetch(self, layer, ids=None, compute_stream=None):
        return _lib.expert_cache_prefetch(self.handle, layer, ids, compute_stream)

    def key_source(self, layer, expert):
        """Index of the stored blob behind key (layer, expert)."""
        E = self.n_experts
        return layer * E + expert if self.store.alias is None else self.store.alias(layer, expert)

    def bandwidth(self):
        """(GB/s, samples): the host-to-device rate the cache's copies achieved."""
        return _lib.expert_cache_bandwidth(self.handle)

    def evict(self, layer, ids=None):
        return _lib.expert_cache_evict(self.handle, layer, ids)

    def stats(self):
        return _lib.expert_cache_stats(self.handle)

    def slots(self):
        return _lib.expert_cache_slots(self.handle)

    def resize(self, pool_bytes, in_place=False, compute_stream=None):
        """Give the cache a pool of `pool_bytes` without reloading from the host:
        in place (shrink, or grow within the allocated pool) or into a new pool
        tensor, after which the old one is released once the copy stream has
        read it. Returns the number of experts moved. Tables from earlier
        prefetch calls are invalid afterwards."""
        import torch
        nbytes = pool_bytes // self.slot_bytes * self.slot_bytes
        if in_place:
            if nbytes > self.pool.numel():
                raise ValueError("in-place growth beyond the allocated pool")
            new = self.pool
        else:
            new = torch.empty(nbytes, dtype=torch.uint8, device=self.pool.device)
        moved = _lib.expert_cache_resize(self.handle, new, nbytes, compute_stream)
        if not in_place:
            self.pool.record_stream(self.copy_stream)   # read by the migration copies
            self.pool = new
        return moved

    def slot_of(self, layer, expert):
        return _lib.expert_cache_slot_of(self.handle, layer, expert)

    def slot_bytes_view(self, slot: int, nbytes: int):
        return self.pool[slot * self.slot_bytes: slot * self.slot_bytes + nbytes]

    def close(self):
        if self.handle:
            _lib.expert_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
