"""Host-side checks of the HIP library (no GPU needed): it loads, exports every
symbol the header declares, and rejects bad arguments before touching the
device."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    from mixture_experts_gate_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_gate_amd import build
        build.build()
    return _lib


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(moe_\w+|expert_cache_\w+)\s*\(", src)
    return sorted(set(names))


def test_header_declares_binding_exports(lib):
    assert _declared_functions() == sorted(lib.EXPORTS)


def test_library_exports_every_symbol(lib):
    L = C.CDLL(lib.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_strerror_and_options(lib):
    L = lib.load()
    assert L.moe_strerror(0) == b"ok"
    assert L.moe_strerror(lib.MOE_EINVAL) == b"invalid argument"
    assert L.moe_strerror(-99) == b"unknown error"
    assert L.moe_get_option(lib.MOE_OPT_FFN_PATH) == 0
    assert L.moe_set_option(lib.MOE_OPT_FFN_PATH, 3) == lib.MOE_EINVAL
    assert L.moe_set_option(99, 0) == lib.MOE_EINVAL


def test_workspace_sizes(lib):
    pb, fb = lib.moe_workspace_size(64, 8, 2048, 768, 128)
    assert pb == 0                      # one-workgroup permutation needs no workspace
    assert fb >= 64 * 8 * 768 * 2
    pb, fb = lib.moe_workspace_size(8192, 8, 2048, 768, 128)
    assert pb >= (64 * 128 + 65536) * 4
    assert fb >= 65536 * 768 * 2
    # tiled path: two FP8 terms + block scales of the activation and of x, and
    # the token-tile map (at most n_pairs / 128 + E tiles)
    assert fb >= (2 * 65536 * 768 + 65536 * 768 // 32 + 2 * 8192 * 2048 + 8192 * 2048 // 32
                  + (65536 // 128 + 128 + 1) * 4)
    with pytest.raises(lib.MoeError):
        lib.moe_workspace_size(-1, 8, 2048, 768, 128)


def test_argument_errors_before_any_device_work(lib):
    L = lib.load()
    dummy = 0x1000  # never dereferenced: validation fails first
    # k > E
    assert L.moe_route(None, None, dummy, None, 4, 64, 8, 9, 1, dummy, dummy, None) == lib.MOE_EINVAL
    # gate needs H % 8 == 0
    assert L.moe_route(dummy, dummy, None, None, 4, 12, 8, 2, 1, dummy, dummy, None) == lib.MOE_EINVAL
    # E above the permutation's limit
    assert L.moe_permute(dummy, 4, 2, 513, dummy, dummy, dummy, None, 0, None) == lib.MOE_EINVAL
    # H not a multiple of 32
    assert L.moe_expert_ffn(dummy, dummy, dummy, dummy, 1, 4, 2, 48, 64, 8, dummy, 0, dummy,
                            1 << 20, None) == lib.MOE_EINVAL
    # workspace too small
    assert L.moe_expert_ffn(dummy, dummy, dummy, dummy, 1, 4, 2, 64, 64, 8, dummy, 0, dummy,
                            16, None) == lib.MOE_EINVAL
    # more experts than the FFN supports
    assert L.moe_expert_ffn(dummy, dummy, dummy, dummy, 1, 4, 2, 128, 128, 513, dummy, 0, dummy,
                            1 << 30, None) == lib.MOE_EINVAL
    # packing: unknown format, K not a multiple of 128, null pointers
    assert L.moe_pack_weights(0, dummy, dummy, 1, 1 << 20, 1 << 20, 256, 256, 0, 0, 0, 0,
                              None) == lib.MOE_EINVAL
    assert L.moe_pack_weights(2, dummy, dummy, 1, 1 << 20, 1 << 20, 256, 192, 0, 0, 0, 0,
                              None) == lib.MOE_EINVAL
    assert L.moe_pack_weights(3, None, dummy, 1, 1 << 20, 1 << 20, 256, 256, 0, 0, 0, 0,
                              None) == lib.MOE_EINVAL
    assert L.moe_pack_weights(3, None, None, 0, 0, 0, 256, 256, 0, 0, 0, 0, None) == lib.MOE_OK
    # NVFP4 / FP8 FFN calls need H, I multiples of 128
    assert L.moe_expert_ffn(dummy, dummy, dummy, dummy, 2, 4, 2, 192, 128, 8, dummy, 0, dummy,
                            1 << 30, None) == lib.MOE_EINVAL
    # bad weight format
    assert L.moe_expert_ffn(dummy, dummy, dummy, dummy, 7, 4, 2, 64, 64, 8, dummy, 0, dummy,
                            1 << 20, None) == lib.MOE_EINVAL
    # combine: H % 8
    assert L.moe_combine(dummy, 0, dummy, None, 4, 2, 12, dummy, None) == lib.MOE_EINVAL
    # T == 0 is a no-op that succeeds
    assert L.moe_combine(None, 0, None, None, 0, 2, 64, None, None) == lib.MOE_OK
    assert L.moe_route(None, None, None, None, 0, 64, 8, 2, 1, None, None, None) == lib.MOE_OK


def test_ffn_shared_argument_errors(lib):
    """moe_expert_ffn_shared: a missing shared expert, a workspace sized for the
    routed rows only and too many experts are refused before device work."""
    L = lib.load()
    dummy = 0x1000  # never dereferenced: validation fails first
    T, k, H, I, E = 8, 4, 256, 128, 16
    _, fb_k = lib.moe_workspace_size(T, k, H, I, E)
    _, fb_k1 = lib.moe_workspace_size(T, k + 1, H, I, E)
    assert fb_k1 > fb_k
    assert L.moe_expert_ffn_shared(dummy, dummy, dummy, dummy, None, 1, T, k, H, I, E, dummy, 0,
                                   dummy, fb_k1, None) == lib.MOE_EINVAL
    assert L.moe_expert_ffn_shared(dummy, dummy, dummy, dummy, dummy, 1, T, k, H, I, E, dummy, 0,
                                   dummy, fb_k, None) == lib.MOE_EINVAL
    assert L.moe_expert_ffn_shared(dummy, dummy, dummy, dummy, dummy, 1, T, k, H, I, 513, dummy,
                                   0, dummy, 1 << 30, None) == lib.MOE_EINVAL
    assert L.moe_expert_ffn_shared(None, None, None, None, None, 1, 0, k, H, I, E, None, 0, None,
                                   0, None) == lib.MOE_OK


def test_ffn_combine_argument_errors(lib):
    """moe_expert_ffn_combine: missing router weights or outputs, a workspace
    sized without the shared expert's rows and a bad format are refused
    before device work; T == 0 succeeds."""
    L = lib.load()
    dummy = 0x1000  # never dereferenced: validation fails first
    T, k, H, I, E = 4, 4, 256, 128, 16
    _, fb_k = lib.moe_workspace_size(T, k, H, I, E)
    _, fb_k1 = lib.moe_workspace_size(T, k + 1, H, I, E)
    args = lambda shared, fmt, tw, y, out, wsb: (dummy, dummy, dummy, dummy, shared, fmt, T, k, H,
                                                 I, E, tw, y, out, dummy, wsb, None)
    assert L.moe_expert_ffn_combine(*args(None, 1, None, dummy, dummy, fb_k)) == lib.MOE_EINVAL
    assert L.moe_expert_ffn_combine(*args(None, 1, dummy, None, dummy, fb_k)) == lib.MOE_EINVAL
    assert L.moe_expert_ffn_combine(*args(None, 1, dummy, dummy, None, fb_k)) == lib.MOE_EINVAL
    assert L.moe_expert_ffn_combine(*args(dummy, 1, dummy, dummy, dummy, fb_k)) == lib.MOE_EINVAL
    assert L.moe_expert_ffn_combine(*args(None, 9, dummy, dummy, dummy, fb_k1)) == lib.MOE_EINVAL
    assert L.moe_expert_ffn_combine(None, None, None, None, None, 1, 0, k, H, I, E, None, None,
                                    None, None, 0, None) == lib.MOE_OK


def test_permute_ffn_combine_argument_errors(lib):
    """moe_permute_ffn_combine: missing offsets, ids, permutation outputs or
    router weights, a workspace sized without the shared expert's rows, too
    many experts and a bad format are refused before device work."""
    L = lib.load()
    dummy = 0x1000  # never dereferenced: validation fails first
    T, k, H, I, E = 8, 4, 256, 128, 16
    _, fb_k = lib.moe_workspace_size(T, k, H, I, E)
    _, fb_k1 = lib.moe_workspace_size(T, k + 1, H, I, E)

    def call(ids=dummy, tw=dummy, shared=None, fmt=1, E_=E, off=dummy, sp=dummy, pr=dummy,
             wsb=fb_k):
        return L.moe_permute_ffn_combine(dummy, ids, tw, dummy, shared, fmt, T, k, H, I, E_, off,
                                         sp, pr, dummy, dummy, dummy, wsb, None)
    assert call(off=None) == lib.MOE_EINVAL
    assert call(ids=None) == lib.MOE_EINVAL
    assert call(tw=None) == lib.MOE_EINVAL
    assert call(sp=None) == lib.MOE_EINVAL
    assert call(pr=None) == lib.MOE_EINVAL
    assert call(shared=dummy) == lib.MOE_EINVAL          # workspace without the shared rows
    assert call(fmt=9, wsb=fb_k1) == lib.MOE_EINVAL
    assert call(E_=513, wsb=1 << 30) == lib.MOE_EINVAL


def test_layer_fused_argument_errors(lib):
    """moe_layer_fused: missing logits, outputs or sync buffer, a misaligned
    sync buffer, a workspace too small or T = 0 are refused (MOE_EINVAL), and
    batches outside the one-launch sizes are declined (MOE_EUNSUPPORTED), both
    before any device work."""
    L = lib.load()
    dummy = 0x1000  # never dereferenced: validation fails first
    T, k, H, I, E = 1, 8, 2048, 768, 128
    _, fb = lib.moe_workspace_size(T, k, H, I, E)

    def call(T_=T, k_=k, H_=H, I_=I, E_=E, fmt=1, lg=dummy, out=dummy, sync=dummy, wsb=fb,
             shared=None):
        return L.moe_layer_fused(dummy, lg, dummy, shared, fmt, T_, k_, H_, I_, E_, 1, dummy,
                                 dummy, dummy, dummy, dummy, dummy, out, dummy, wsb, sync, None)
    assert call(lg=None) == lib.MOE_EINVAL
    assert call(out=None) == lib.MOE_EINVAL
    assert call(sync=None) == lib.MOE_EINVAL
    assert call(sync=dummy + 4) == lib.MOE_EINVAL            # not 8-byte aligned
    assert call(wsb=fb - 1) == lib.MOE_EINVAL
    assert call(T_=0) == lib.MOE_EINVAL
    assert call(k_=200) == lib.MOE_EINVAL                    # k > E
    big = 1 << 30
    assert call(T_=4, wsb=big) == lib.MOE_EUNSUPPORTED       # 32 rows
    assert call(T_=9, k_=1, wsb=big) == lib.MOE_EUNSUPPORTED  # more tokens than wavefronts
    assert call(E_=300, wsb=big) == lib.MOE_EUNSUPPORTED     # ids past 8 bits
    assert call(fmt=0, wsb=big) == lib.MOE_EUNSUPPORTED      # bf16 weights
    assert call(H_=1536, wsb=big) == lib.MOE_EUNSUPPORTED    # 12 slabs of gate/up
    assert call(I_=1024, wsb=big) == lib.MOE_EUNSUPPORTED    # 8 slabs of down
    assert call(shared=dummy, k_=7, T_=4, wsb=big) == lib.MOE_EUNSUPPORTED  # 32 rows


def test_cache_reserve_argument_errors(lib):
    L = lib.load()
    h = C.c_void_p(0)
    src = (C.c_void_p * 2)(0x1000, 0x2000)
    # pool too small for one layer of experts
    assert L.expert_cache_reserve(C.byref(h), 0x1000, 1024, 1024, 1, 2, src, 0, 0, 0, 0,
                                  None) == lib.MOE_ENOMEM
    # null host source
    src0 = (C.c_void_p * 2)(0x1000, None)
    assert L.expert_cache_reserve(C.byref(h), 0x1000, 1 << 20, 1024, 1, 2, src0, 0, 0, 0, 0,
                                  None) == lib.MOE_EINVAL
    assert L.expert_cache_destroy(None) == lib.MOE_EINVAL
    assert L.expert_cache_slots(None) == lib.MOE_EINVAL
    assert L.expert_cache_resize(None, 0x1000, 1 << 20, None, None) == lib.MOE_EINVAL
