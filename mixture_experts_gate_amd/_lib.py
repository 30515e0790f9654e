"""ctypes binding of ``libmoe.so`` (the C ABI in include/moe.h).

Argument marshalling only: tensors become raw device pointers, streams become
hipStream_t handles, and every return code is turned into an exception. All of
the layer's work runs in the HIP kernels of the library. There is no fallback:
if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOMEM, MOE_EHIP, MOE_EUNSUPPORTED, MOE_EBUSY = 0, -1, -2, -3, -4, -5
MOE_W_BF16, MOE_W_MXFP4, MOE_W_NVFP4, MOE_W_FP8 = 0, 1, 2, 3
MOE_OPT_FFN_PATH = 1
MOE_OPT_TIMING = 2
MOE_OPT_DEC_SPLIT = 3
MOE_OPT_CACHE_FAULT = 4
MOE_OPT_CACHE_DELAY_US = 5
MOE_OPT_CACHE_THROTTLE_MBS = 6
MOE_OPT_PRE_GROUP = 7

# every symbol include/moe.h declares
EXPORTS = [
    "moe_strerror", "moe_last_hip_error", "moe_route", "moe_permute", "moe_expert_ffn",
    "moe_expert_ffn_shared", "moe_expert_ffn_noalloc", "moe_expert_ffn_combine",
    "moe_combine", "moe_workspace_size", "moe_set_option", "moe_get_option", "moe_kernel_name",
    "moe_timing_query", "moe_pack_mxfp4", "moe_pack_weights", "moe_route_permute",
    "expert_cache_reserve", "expert_cache_prefetch", "expert_cache_evict", "expert_cache_stats",
    "expert_cache_slots", "expert_cache_slot_of", "expert_cache_destroy", "expert_cache_resize",
    "moe_micro_read", "moe_micro_mfma", "expert_cache_bandwidth", "expert_cache_prefetch_qstar",
    "moe_permute_split", "moe_cpu_expert_ffn", "moe_scatter_rows", "moe_permute_ffn_combine",
    "moe_layer_fused",
]


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str, hip: int):
        super().__init__(f"{fn} failed: {text} ({code})" + (f", hip error {hip}" if code == MOE_EHIP else ""))
        self.code = code
        self.hip = hip


class ExpertW(C.Structure):
    """moe_expert_w"""
    _fields_ = [("w13", C.c_void_p), ("s13", C.c_void_p), ("w2", C.c_void_p), ("s2", C.c_void_p)]


_lib = None


def load(path: str | None = None):
    """Load the library (raises if it is not built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run __graft_entry__.build() or "
                           "python -m mixture_experts_gate_amd.build")
    L = C.CDLL(p)
    P, I, Z = C.c_void_p, C.c_int, C.c_size_t
    sig = {
        "moe_strerror": (C.c_char_p, [I]),
        "moe_last_hip_error": (I, []),
        "moe_route": (I, [P, P, P, P, I, I, I, I, I, P, P, P]),
        "moe_permute": (I, [P, I, I, I, P, P, P, P, Z, P]),
        "moe_route_permute": (I, [P, P, P, P, I, I, I, I, I, P, P, P, P, P, P, Z, P]),
        "moe_expert_ffn": (I, [P, P, P, P, I, I, I, I, I, I, P, I, P, Z, P]),
        "moe_expert_ffn_shared": (I, [P, P, P, P, P, I, I, I, I, I, I, P, I, P, Z, P]),
        "moe_expert_ffn_noalloc": (I, [P, P, P, P, I, I, I, I, I, I, P, I, P]),
        "moe_expert_ffn_combine": (I, [P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, Z, P]),
        "moe_permute_ffn_combine": (I, [P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P, P, Z,
                                        P]),
        "moe_layer_fused": (I, [P, P, P, P, I, I, I, I, I, I, I, P, P, P, P, P, P, P, P, Z, P,
                                P]),
        "moe_combine": (I, [P, I, P, P, I, I, I, P, P]),
        "moe_workspace_size": (I, [I, I, I, I, I, C.POINTER(Z), C.POINTER(Z)]),
        "moe_set_option": (I, [I, I]),
        "moe_get_option": (I, [I]),
        "moe_kernel_name": (C.c_char_p, [I]),
        "moe_timing_query": (I, [I, C.POINTER(C.c_longlong), C.POINTER(C.c_double)]),
        "moe_pack_mxfp4": (I, [P, P, I, Z, Z, I, I, Z, Z, Z, Z, P]),
        "moe_pack_weights": (I, [I, P, P, I, Z, Z, I, I, Z, Z, Z, Z, P]),
        "expert_cache_reserve": (I, [C.POINTER(P), P, Z, Z, I, I, P, Z, Z, Z, Z, P]),
        "expert_cache_prefetch": (I, [P, I, P, I, P, C.POINTER(P)]),
        "expert_cache_evict": (I, [P, I, P, I]),
        "expert_cache_resize": (I, [P, P, Z, P, C.POINTER(I)]),
        "expert_cache_stats": (I, [P, C.POINTER(C.c_longlong), C.POINTER(C.c_longlong),
                                   C.POINTER(C.c_longlong)]),
        "expert_cache_slots": (I, [P]),
        "expert_cache_slot_of": (I, [P, I, I]),
        "expert_cache_destroy": (I, [P]),
        "moe_micro_read": (I, [P, Z, I, P, P]),
        "moe_micro_mfma": (I, [I, I, I, P, C.POINTER(C.c_double), P]),
        "expert_cache_bandwidth": (I, [P, C.POINTER(C.c_double), C.POINTER(C.c_longlong)]),
        "expert_cache_prefetch_qstar": (I, [P, I, P, P, I, C.c_double, C.c_double, C.c_double,
                                            C.c_double, P, C.POINTER(P), P, C.POINTER(I)]),
        "moe_permute_split": (I, [P, P, I, P, P, P, P, C.POINTER(I)]),
        "moe_cpu_expert_ffn": (I, [I, P, P, P, P, I, I, P, I, P, I]),
        "moe_scatter_rows": (I, [P, P, I, Z, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = L
    return L


def _check(fn: str, rc: int) -> int:
    if rc < 0:
        L = load()
        raise MoeError(fn, rc, L.moe_strerror(rc).decode(), L.moe_last_hip_error())
    return rc


def _ptr(t):
    """Device (or host) address of a tensor, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------- layer calls --

def moe_route(x_bf16, wg_bf16, logits_in, logits_out, T, H, E, k, renormalize, topk_ids, topk_w,
              stream=None):
    return _check("moe_route", load().moe_route(
        _ptr(x_bf16), _ptr(wg_bf16), _ptr(logits_in), _ptr(logits_out), T, H, E, k,
        int(bool(renormalize)), _ptr(topk_ids), _ptr(topk_w), _stream(stream)))


def moe_permute(topk_ids, T, k, E, offsets, sorted_pair, pair_row, ws, ws_bytes, stream=None):
    return _check("moe_permute", load().moe_permute(
        _ptr(topk_ids), T, k, E, _ptr(offsets), _ptr(sorted_pair), _ptr(pair_row), _ptr(ws),
        ws_bytes, _stream(stream)))


def moe_route_permute(x_bf16, wg_bf16, logits_in, logits_out, T, H, E, k, renormalize, topk_ids,
                      topk_w, offsets, sorted_pair, pair_row, ws, ws_bytes, stream=None):
    return _check("moe_route_permute", load().moe_route_permute(
        _ptr(x_bf16), _ptr(wg_bf16), _ptr(logits_in), _ptr(logits_out), T, H, E, k,
        int(bool(renormalize)), _ptr(topk_ids), _ptr(topk_w), _ptr(offsets), _ptr(sorted_pair),
        _ptr(pair_row), _ptr(ws), ws_bytes, _stream(stream)))


def moe_expert_ffn(x_bf16, sorted_pair, offsets, experts, fmt, T, k, H, I, E, y, y_is_fp32, ws,
                   ws_bytes, stream=None):
    return _check("moe_expert_ffn", load().moe_expert_ffn(
        _ptr(x_bf16), _ptr(sorted_pair), _ptr(offsets), _ptr(experts), fmt, T, k, H, I, E, _ptr(y),
        int(bool(y_is_fp32)), _ptr(ws), ws_bytes, _stream(stream)))


def moe_expert_ffn_shared(x_bf16, sorted_pair, offsets, experts, shared, fmt, T, k, H, I, E, y,
                          y_is_fp32, ws, ws_bytes, stream=None, check=True):
    """Routed + shared expert FFN in the same launches (y has T*k + T rows).
    check=False returns MOE_EUNSUPPORTED instead of raising, so that the
    caller can run the shared expert as its own call on the tiled path."""
    rc = load().moe_expert_ffn_shared(
        _ptr(x_bf16), _ptr(sorted_pair), _ptr(offsets), _ptr(experts), _ptr(shared), fmt, T, k, H,
        I, E, _ptr(y), int(bool(y_is_fp32)), _ptr(ws), ws_bytes, _stream(stream))
    if not check and rc == MOE_EUNSUPPORTED:
        return rc
    return _check("moe_expert_ffn_shared", rc)


def moe_expert_ffn_combine(x_bf16, sorted_pair, offsets, experts, shared, fmt, T, k, H, I, E,
                           topk_w, y, out, ws, ws_bytes, stream=None, check=True):
    """Expert FFN (with the shared expert when `shared` is given) and the
    weighted combine into `out`; y (bf16) holds the expert rows. check=False
    returns MOE_EUNSUPPORTED instead of raising."""
    rc = load().moe_expert_ffn_combine(
        _ptr(x_bf16), _ptr(sorted_pair), _ptr(offsets), _ptr(experts), _ptr(shared), fmt, T, k, H,
        I, E, _ptr(topk_w), _ptr(y), _ptr(out), _ptr(ws), ws_bytes, _stream(stream))
    if not check and rc == MOE_EUNSUPPORTED:
        return rc
    return _check("moe_expert_ffn_combine", rc)


def moe_permute_ffn_combine(x_bf16, topk_ids, topk_w, experts, shared, fmt, T, k, H, I, E,
                            offsets, sorted_pair, pair_row, y, out, ws, ws_bytes, stream=None):
    """The permutation of the router's ids, the expert FFN (with the shared
    expert when `shared` is given) and the weighted combine into `out`."""
    _check("moe_permute_ffn_combine", load().moe_permute_ffn_combine(
        _ptr(x_bf16), _ptr(topk_ids), _ptr(topk_w), _ptr(experts), _ptr(shared), fmt, T, k, H, I,
        E, _ptr(offsets), _ptr(sorted_pair), _ptr(pair_row), _ptr(y), _ptr(out), _ptr(ws),
        ws_bytes, _stream(stream)))


def moe_layer_fused(x_bf16, logits, experts, shared, fmt, T, k, H, I, E, renormalize, topk_ids,
                    topk_w, offsets, sorted_pair, pair_row, y, out, ws, ws_bytes, sync,
                    stream=None, check=True):
    """The whole layer from given logits in one launch (a handful of tokens);
    sync: LAYER_SYNC_BYTES of zero-initialised device memory (the calls keep
    it consistent). check=False returns MOE_EUNSUPPORTED instead of raising."""
    rc = load().moe_layer_fused(
        _ptr(x_bf16), _ptr(logits), _ptr(experts), _ptr(shared), fmt, T, k, H, I, E,
        int(bool(renormalize)), _ptr(topk_ids), _ptr(topk_w), _ptr(offsets), _ptr(sorted_pair),
        _ptr(pair_row), _ptr(y), _ptr(out), _ptr(ws), ws_bytes, _ptr(sync), _stream(stream))
    if not check and rc == MOE_EUNSUPPORTED:
        return rc
    return _check("moe_layer_fused", rc)


LAYER_SYNC_BYTES = 8192      # MOE_LAYER_SYNC_BYTES

FFN_NOALLOC_MAX_WS = 64 << 20


def moe_expert_ffn_noalloc(x_bf16, sorted_pair, offsets, experts, fmt, T, k, H, I, E, y,
                           y_is_fp32, stream=None):
    """moe_expert_ffn with the library's own per-device workspace array."""
    return _check("moe_expert_ffn_noalloc", load().moe_expert_ffn_noalloc(
        _ptr(x_bf16), _ptr(sorted_pair), _ptr(offsets), _ptr(experts), fmt, T, k, H, I, E, _ptr(y),
        int(bool(y_is_fp32)), _stream(stream)))


def moe_combine(y, y_is_fp32, topk_w, y_shared, T, k, H, out_bf16, stream=None):
    return _check("moe_combine", load().moe_combine(
        _ptr(y), int(bool(y_is_fp32)), _ptr(topk_w), _ptr(y_shared), T, k, H, _ptr(out_bf16),
        _stream(stream)))


def moe_pack_mxfp4(src, dst, n, src_stride, dst_stride, H, I, layout, stream=None):
    return _check("moe_pack_mxfp4", load().moe_pack_mxfp4(
        _ptr(src), _ptr(dst), n, src_stride, dst_stride, H, I, layout.w13, layout.s13, layout.w2,
        layout.s2, _stream(stream)))


def moe_pack_weights(fmt, src, dst, n, src_stride, dst_stride, H, I, layout, stream=None):
    return _check("moe_pack_weights", load().moe_pack_weights(
        fmt, _ptr(src), _ptr(dst), n, src_stride, dst_stride, H, I, layout.w13, layout.s13,
        layout.w2, layout.s2, _stream(stream)))


def moe_workspace_size(T, k, H, I, E):
    a, b = C.c_size_t(0), C.c_size_t(0)
    _check("moe_workspace_size", load().moe_workspace_size(T, k, H, I, E, C.byref(a), C.byref(b)))
    return a.value, b.value


def moe_set_option(option, value):
    return _check("moe_set_option", load().moe_set_option(option, value))


def moe_get_option(option):
    return _check("moe_get_option", load().moe_get_option(option))


def kernel_names():
    L = load()
    out = []
    i = 0
    while True:
        n = L.moe_kernel_name(i)
        if n is None:
            return out
        out.append(n.decode())
        i += 1


def moe_timing_query(kernel_id):
    """(launches, total_ms) of one kernel since timing was last switched."""
    n, ms = C.c_longlong(0), C.c_double(0.0)
    _check("moe_timing_query", load().moe_timing_query(kernel_id, C.byref(n), C.byref(ms)))
    return n.value, ms.value


def timing_report():
    """{kernel name: (launches, total_ms)} for kernels launched while timing was on."""
    rep = {}
    for i, name in enumerate(kernel_names()):
        n, ms = moe_timing_query(i)
        if n:
            rep[name] = (n, ms)
    return rep


# ------------------------------------------------------- measurement helpers --

def moe_micro_read(buf, nbytes, grid, sink, stream=None):
    return _check("moe_micro_read", load().moe_micro_read(_ptr(buf), nbytes, grid, _ptr(sink),
                                                          _stream(stream)))


def moe_micro_mfma(kind, grid, iters, sink, stream=None):
    """Returns the FLOPs of the launch."""
    f = C.c_double(0.0)
    _check("moe_micro_mfma", load().moe_micro_mfma(kind, grid, iters, _ptr(sink), C.byref(f),
                                                   _stream(stream)))
    return f.value


# ------------------------------------------------------------ expert cache --

def expert_cache_reserve(pool, pool_bytes, expert_bytes, n_layers, n_experts, host_src, layout,
                         copy_stream):
    """host_src: sequence of host addresses (ints) of pinned blobs, [L*E]."""
    h = C.c_void_p(0)
    arr = (C.c_void_p * len(host_src))(*host_src)
    _check("expert_cache_reserve", load().expert_cache_reserve(
        C.byref(h), _ptr(pool), pool_bytes, expert_bytes, n_layers, n_experts, arr,
        layout.w13, layout.s13, layout.w2, layout.s2, _stream(copy_stream)))
    return h.value


def expert_cache_prefetch(cache, layer, ids, compute_stream=None):
    """ids: host int32 numpy array or None (whole layer). Returns the device table address."""
    tab = C.c_void_p(0)
    if ids is None:
        p, n = None, 0
    else:
        import numpy as np
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        p, n = ids.ctypes.data_as(C.c_void_p), int(ids.size)
    _check("expert_cache_prefetch", load().expert_cache_prefetch(
        cache, layer, p, n, _stream(compute_stream), C.byref(tab)))
    return tab.value


def expert_cache_evict(cache, layer, ids=None):
    if ids is None:
        p, n = None, 0
    else:
        import numpy as np
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        p, n = ids.ctypes.data_as(C.c_void_p), int(ids.size)
    return _check("expert_cache_evict", load().expert_cache_evict(cache, layer, p, n))


def expert_cache_stats(cache):
    h, m, b = C.c_longlong(0), C.c_longlong(0), C.c_longlong(0)
    _check("expert_cache_stats", load().expert_cache_stats(cache, C.byref(h), C.byref(m), C.byref(b)))
    return h.value, m.value, b.value


def expert_cache_resize(cache, new_pool, new_pool_bytes, compute_stream=None):
    """Move the cache to `new_pool` (tensor or address); returns the number of
    experts copied device to device."""
    moved = C.c_int(0)
    _check("expert_cache_resize", load().expert_cache_resize(
        cache, _ptr(new_pool), new_pool_bytes, _stream(compute_stream), C.byref(moved)))
    return moved.value


def expert_cache_bandwidth(cache):
    """(GB/s, samples) of the cache's measured host-to-device rate."""
    g, n = C.c_double(0.0), C.c_longlong(0)
    _check("expert_cache_bandwidth", load().expert_cache_bandwidth(cache, C.byref(g), C.byref(n)))
    return g.value, n.value


def expert_cache_prefetch_qstar(cache, layer, ids, rows, host_s_fixed, host_s_per_expert,
                                host_s_per_row, n_experts, link_gbs=0.0, compute_stream=None):
    """Returns (device table address, host mask uint8 [n_experts])."""
    import numpy as np
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    mask = np.zeros(n_experts, dtype=np.uint8)
    tab, nh = C.c_void_p(0), C.c_int(0)
    _check("expert_cache_prefetch_qstar", load().expert_cache_prefetch_qstar(
        cache, layer, ids.ctypes.data_as(C.c_void_p), rows.ctypes.data_as(C.c_void_p),
        int(ids.size), float(host_s_fixed), float(host_s_per_expert), float(host_s_per_row),
        float(link_gbs),
        _stream(compute_stream),
        C.byref(tab), mask.ctypes.data_as(C.c_void_p), C.byref(nh)))
    return tab.value, mask


def moe_permute_split(offsets, sorted_pair, host_mask):
    """Host arrays -> (dev_offsets, dev_sorted_pair, host_pairs) as numpy int32."""
    import numpy as np
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    sp = np.ascontiguousarray(sorted_pair, dtype=np.int32)
    mask = np.ascontiguousarray(host_mask, dtype=np.uint8)
    E = off.size - 1
    n = int(off[-1])
    d_off = np.empty(E + 1, dtype=np.int32)
    d_sp = np.empty(max(n, 1), dtype=np.int32)
    h_p = np.empty(max(n, 1), dtype=np.int32)
    nh = C.c_int(0)
    _check("moe_permute_split", load().moe_permute_split(
        off.ctypes.data_as(C.c_void_p), sp.ctypes.data_as(C.c_void_p), E,
        mask.ctypes.data_as(C.c_void_p), d_off.ctypes.data_as(C.c_void_p),
        d_sp.ctypes.data_as(C.c_void_p), h_p.ctypes.data_as(C.c_void_p), C.byref(nh)))
    return d_off, d_sp[:int(d_off[-1])], h_p[:nh.value]


def moe_cpu_expert_ffn(fmt, w13, s13, w2, s2, H, I, x_rows, y_rows, threads=0):
    """x_rows, y_rows: host numpy uint16 [n][H] (y written in place); weight
    pointers: host addresses."""
    n = int(x_rows.shape[0])
    return _check("moe_cpu_expert_ffn", load().moe_cpu_expert_ffn(
        fmt, w13, s13, w2, s2, H, I, x_rows.ctypes.data_as(C.c_void_p), n,
        y_rows.ctypes.data_as(C.c_void_p), threads))


def moe_scatter_rows(src, idx, n, row_bytes, dst, stream=None):
    return _check("moe_scatter_rows", load().moe_scatter_rows(
        _ptr(src), _ptr(idx), n, row_bytes, _ptr(dst), _stream(stream)))


def expert_cache_slots(cache):
    return _check("expert_cache_slots", load().expert_cache_slots(cache))


def expert_cache_slot_of(cache, layer, expert):
    return load().expert_cache_slot_of(cache, layer, expert)


def expert_cache_destroy(cache):
    return _check("expert_cache_destroy", load().expert_cache_destroy(cache))
