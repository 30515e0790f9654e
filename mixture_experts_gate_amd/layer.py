"""Device-side orchestration of one MoE layer on top of the C ABI.

PyTorch only provides device memory and the stream; every step of the layer
(routing, permutation, expert FFN, combine, cache copies) is a call into
``libmoe.so``. Buffers are allocated once per (layer shape, max T) and reused.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib
from .synth import blob_layout

FMT = {"bf16": _lib.MOE_W_BF16, "mxfp4": _lib.MOE_W_MXFP4}


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
    device tensor of the same shape in the kernel layout (MXFP4 blocks packed
    by the library; bf16 blobs are used as they are)."""
    host = torch.from_numpy(np.ascontiguousarray(pool, dtype=np.uint8))
    if host.dim() == 1:
        host = host[None, :]
    src = host.to(device)
    if layout.fmt != "mxfp4":
        return src
    dst = torch.empty_like(src)
    n, nb = src.shape
    _lib.moe_pack_mxfp4(src, dst, n, nb, nb, layout.H, layout.I, layout)
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
        pb, fb = _lib.moe_workspace_size(T_max, k, H, I, E)
        self.ws_perm_bytes = max(pb, 256)
        self.ws_ffn_bytes = fb
        self.ws_perm = torch.empty(self.ws_perm_bytes, dtype=torch.uint8, device=dev)
        self.ws_ffn = torch.empty(fb, dtype=torch.uint8, device=dev)
        self.y = torch.empty((max(n, 1), H), dtype=ydt, device=dev)
        self.out = torch.empty((T_max, H), dtype=torch.bfloat16, device=dev)
        if shared:
            self.sh_pair = torch.arange(T_max, dtype=torch.int32, device=dev)
            self.sh_off = torch.empty(2, dtype=torch.int32, device=dev)
            _, fbs = _lib.moe_workspace_size(T_max, 1, H, I, 1)
            self.ws_sh_bytes = fbs
            self.ws_sh = torch.empty(fbs, dtype=torch.uint8, device=dev)
            self.y_sh = torch.empty((T_max, H), dtype=ydt, device=dev)
        self._sh_T = -1

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

    def ffn(self, T, x, table, stream=None):
        _lib.moe_expert_ffn(x, self.sorted_pair, self.offsets, table, self.fmt, T, self.k, self.H,
                            self.I, self.E, self.y, self.y_fp32, self.ws_ffn, self.ws_ffn_bytes,
                            stream)

    def combine(self, T, with_shared=False, stream=None):
        _lib.moe_combine(self.y, self.y_fp32, self.topk_w, self.y_sh if with_shared else None, T,
                         self.k, self.H, self.out, stream)

    # whole layer -----------------------------------------------------------
    def forward(self, T, x, table, logits=None, wg=None, shared_table=None, renormalize=True,
                stream=None, write_logits=False, fused_routing=True):
        """route -> permute -> expert FFN (+ shared expert) -> combine; returns out[:T].
        fused_routing: route and permute with the one-call entry (one kernel for
        small batches) instead of the two separate calls."""
        if T > self.T_max:
            raise ValueError("T exceeds the buffers' T_max")
        wl = write_logits or logits is None
        if fused_routing:
            self.route_permute(T, x=x, wg=wg, logits=logits, renormalize=renormalize,
                               stream=stream, write_logits=wl)
        else:
            self.route(T, x=x, wg=wg, logits=logits, renormalize=renormalize, stream=stream,
                       write_logits=wl)
            self.permute(T, stream)
        self.ffn(T, x, table, stream)
        if shared_table is not None:
            if self._sh_T != T:
                self.prepare_shared(T)
            self.shared_ffn(T, x, shared_table, stream)
        self.combine(T, with_shared=shared_table is not None, stream=stream)
        return self.out[:T]

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
