"""CPU oracle for the routed MoE expert layer -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package. The GPU library and its Python binding never do.

``build()`` compiles ``oracle.c`` with gcc (single thread, -O2, no FP
contraction, no fast-math, no vector intrinsics); the functions below marshal
numpy arrays into it. Every function states the definition it follows in
``oracle.c``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(_LIB_PATH)
        P = C.c_void_p
        L.orc_bf16_to_f64.restype = C.c_double
        L.orc_bf16_to_f64.argtypes = [C.c_uint16]
        L.orc_f64_to_bf16.restype = C.c_uint16
        L.orc_f64_to_bf16.argtypes = [C.c_double]
        L.orc_e2m1.restype = C.c_double
        L.orc_e2m1.argtypes = [C.c_int]
        L.orc_e8m0.restype = C.c_double
        L.orc_e8m0.argtypes = [C.c_int]
        L.orc_mxfp4_decode.restype = None
        L.orc_mxfp4_decode.argtypes = [P, P, C.c_long, C.c_long, P]
        L.orc_e4m3.restype = C.c_double
        L.orc_e4m3.argtypes = [C.c_int]
        L.orc_nvfp4_decode.restype = None
        L.orc_nvfp4_decode.argtypes = [P, P, C.c_float, C.c_long, C.c_long, P]
        L.orc_fp8_decode.restype = None
        L.orc_fp8_decode.argtypes = [P, C.c_float, C.c_long, C.c_long, P]
        L.orc_gate_logits_f32.restype = None
        L.orc_gate_logits_f32.argtypes = [P, P, C.c_int, C.c_int, C.c_int, P]
        L.orc_gate_logits_f64.restype = None
        L.orc_gate_logits_f64.argtypes = [P, P, C.c_int, C.c_int, C.c_int, P]
        L.orc_topk.restype = C.c_int
        L.orc_topk.argtypes = [P, C.c_int, C.c_int, C.c_int, C.c_int, P, P, P]
        L.orc_permute.restype = C.c_int
        L.orc_permute.argtypes = [P, C.c_int, C.c_int, C.c_int, P, P, P]
        L.orc_ffn_rows.restype = C.c_int
        L.orc_ffn_rows.argtypes = [P, C.c_int, C.c_int, C.c_int, P, C.c_int, C.c_long, P, P, P, P]
        L.orc_combine.restype = None
        L.orc_combine.argtypes = [P, P, P, C.c_long, C.c_int, C.c_int, P, P]
        L.orc_moe_layer.restype = C.c_int
        L.orc_moe_layer.argtypes = [P, P, P, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                    C.c_int, P, P, P, P, P, P, P, P, P, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ codecs --

def bf16_to_f64(bits) -> float:
    return lib().orc_bf16_to_f64(int(bits))


def f64_to_bf16(v: float) -> int:
    return int(lib().orc_f64_to_bf16(float(v)))


def e2m1(code: int) -> float:
    return lib().orc_e2m1(int(code))


def e8m0(s: int) -> float:
    return lib().orc_e8m0(int(s))


def mxfp4_decode(codes: np.ndarray, scales: np.ndarray, R: int, K: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    out = np.empty((R, K), dtype=np.float64)
    lib().orc_mxfp4_decode(_p(codes), _p(scales), R, K, _p(out))
    return out


def e4m3(code: int) -> float:
    return lib().orc_e4m3(int(code))


def nvfp4_decode(codes: np.ndarray, scales: np.ndarray, g: float, R: int, K: int) -> np.ndarray:
    """Rows [R][K] from E2M1 codes [R][K/2], E4M3 block scales [R][K/16] and the
    matrix's fp32 scale g."""
    out = np.empty((R, K), dtype=np.float64)
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    lib().orc_nvfp4_decode(_p(codes), _p(scales), float(g), R, K, _p(out))
    return out


def fp8_decode(codes: np.ndarray, g: float, R: int, K: int) -> np.ndarray:
    out = np.empty((R, K), dtype=np.float64)
    codes = _c(codes, np.uint8)
    lib().orc_fp8_decode(_p(codes), float(g), R, K, _p(out))
    return out


# ------------------------------------------------------------------ router --

def gate_logits_f32(x: np.ndarray, wg: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint16)
    wg = _c(wg, np.uint16)
    T, H = x.shape
    E = wg.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    lib().orc_gate_logits_f32(_p(x), _p(wg), T, H, E, _p(out))
    return out


def gate_logits_f64(x: np.ndarray, wg: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint16)
    wg = _c(wg, np.uint16)
    T, H = x.shape
    E = wg.shape[0]
    out = np.empty((T, E), dtype=np.float64)
    lib().orc_gate_logits_f64(_p(x), _p(wg), T, H, E, _p(out))
    return out


def topk(logits: np.ndarray, k: int, renormalize: bool = True):
    """Returns (ids int32 [T][k], w fp32 [T][k], w64 double [T][k])."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    w64 = np.empty((T, k), dtype=np.float64)
    rc = lib().orc_topk(_p(lg), T, E, k, int(bool(renormalize)), _p(ids), _p(w), _p(w64))
    if rc != 0:
        raise ValueError("non-finite router logit")
    return ids, w, w64


def permute(ids: np.ndarray, E: int):
    """Returns (offsets [E+1], sorted_pair [T*k], pair_row [T*k]), all int32."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    off = np.empty(E + 1, dtype=np.int32)
    sp = np.empty(T * k, dtype=np.int32)
    pr = np.empty(T * k, dtype=np.int32)
    if lib().orc_permute(_p(ids), T, k, E, _p(off), _p(sp), _p(pr)) != 0:
        raise ValueError("expert id out of range")
    return off, sp, pr


# --------------------------------------------------------------------- FFN --

class _Expert(C.Structure):
    _fields_ = [("w13", C.c_void_p), ("s13", C.c_void_p), ("w2", C.c_void_p), ("s2", C.c_void_p)]


def _expert_table(blobs: np.ndarray, layout):
    """blobs: uint8 [n][nbytes] (one expert per row) in the storage layout."""
    blobs = np.ascontiguousarray(blobs, dtype=np.uint8)
    if blobs.ndim == 1:
        blobs = blobs[None, :]
    base = blobs.ctypes.data
    stride = blobs.strides[0]
    tab = (_Expert * blobs.shape[0])()
    for e in range(blobs.shape[0]):
        b = base + e * stride
        tab[e] = _Expert(b + layout.w13, b + layout.s13, b + layout.w2, b + layout.s2)
    return tab, blobs


def _fmt_code(layout) -> int:
    return {"bf16": 0, "mxfp4": 1, "nvfp4": 2, "fp8": 3}[layout.fmt]


def ffn_rows(x: np.ndarray, blobs: np.ndarray, layout, row_token, row_expert, want_act=False):
    """SwiGLU FFN of expert row_expert[r] on token row_token[r]; returns y [n][H]
    (and the activation [n][I] when want_act)."""
    x = _c(x, np.uint16)
    H, I = layout.H, layout.I
    assert x.shape[1] == H
    tab, keep = _expert_table(blobs, layout)
    rt = _c(row_token, np.int32)
    re = _c(row_expert, np.int32)
    n = rt.shape[0]
    y = np.empty((n, H), dtype=np.float64)
    act = np.empty((n, I), dtype=np.float64) if want_act else None
    rc = lib().orc_ffn_rows(_p(x), H, I, _fmt_code(layout), C.cast(tab, C.c_void_p), len(tab), n,
                            _p(rt), _p(re), _p(y), _p(act))
    del keep
    if rc != 0:
        raise ValueError("orc_ffn_rows failed")
    return (y, act) if want_act else y


def combine(y: np.ndarray, w: np.ndarray, y_shared=None):
    """Returns (out_f64 [T][H], out_bf16 bits [T][H])."""
    w = _c(w, np.float32)
    T, k = w.shape
    y = _c(y, np.float64)
    H = y.shape[1]
    assert y.shape[0] == T * k
    ysh = None if y_shared is None else _c(y_shared, np.float64)
    out = np.empty((T, H), dtype=np.float64)
    ob = np.empty((T, H), dtype=np.uint16)
    lib().orc_combine(_p(y), _p(w), _p(ysh), T, k, H, _p(out), _p(ob))
    return out, ob


def moe_layer(x, layout, blobs, k, logits=None, wg=None, shared_blob=None, renormalize=True):
    """Whole layer for all tokens of x. Returns a dict of every stage's output."""
    x = _c(x, np.uint16)
    T, H = x.shape
    E = blobs.shape[0]
    tab, keep = _expert_table(blobs, layout)
    stab, skeep = (None, None)
    if shared_blob is not None:
        stab, skeep = _expert_table(shared_blob, layout)
    lg = None if logits is None else _c(logits, np.float32)
    wgc = None if wg is None else _c(wg, np.uint16)
    if lg is None and wgc is None:
        raise ValueError("need logits or gate weights")
    r = dict(
        logits=np.empty((T, E), np.float32), ids=np.empty((T, k), np.int32),
        w=np.empty((T, k), np.float32), offsets=np.empty(E + 1, np.int32),
        sorted_pair=np.empty(T * k, np.int32), pair_row=np.empty(T * k, np.int32),
        y=np.empty((T * k, H), np.float64), out_f64=np.empty((T, H), np.float64),
        out_bf16=np.empty((T, H), np.uint16))
    rc = lib().orc_moe_layer(
        _p(x), _p(wgc), _p(lg), T, H, E, k, layout.I, _fmt_code(layout), int(bool(renormalize)),
        C.cast(tab, C.c_void_p), None if stab is None else C.cast(stab, C.c_void_p),
        _p(r["logits"]), _p(r["ids"]), _p(r["w"]), _p(r["offsets"]), _p(r["sorted_pair"]),
        _p(r["pair_row"]), _p(r["y"]), _p(r["out_f64"]), _p(r["out_bf16"]))
    del keep, skeep
    if rc != 0:
        raise ValueError("orc_moe_layer failed")
    return r
