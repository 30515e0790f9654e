// Internal helpers shared by the gfx950 kernels of the MoE layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int kWave = 64;

// ---------------------------------------------------------------- errors --

void set_last_hip_error(hipError_t e);

// Returns MOE_EHIP (and records the code) if a launch failed.
inline int check_launch() {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_last_hip_error(e);
        return MOE_EHIP;
    }
    return MOE_OK;
}

inline int check_hip(hipError_t e) {
    if (e != hipSuccess) {
        set_last_hip_error(e);
        return MOE_EHIP;
    }
    return MOE_OK;
}

int ffn_path_option();
// Expert-cache test knobs (MOE_OPT_CACHE_FAULT, MOE_OPT_CACHE_DELAY_US).
int cache_set_fault(int n);
int cache_get_fault();
int cache_set_delay(int us);
int cache_get_delay();
int cache_set_throttle(int mbs);
int cache_get_throttle();
// Consecutive weight tiles per workgroup of the tiled kernels (MOE_OPT_PRE_GROUP).
int pre_group(int stage);
// Weights of the decode kernels' tile split for stage 1 or 2 (MOE_OPT_DEC_SPLIT).
void dec_split_weights(int stage, float *w_slot, float *w_pos);

// Kernel ids for the optional launch timing (moe_timing_query).
enum KernelId {
    K_ROUTE = 0, K_PERM_SMALL, K_PERM_RANK, K_PERM_SCAN, K_PERM_SCATTER, K_PERM_EMPTY,
    K_DEC_GATE_UP, K_DEC_DOWN, K_PRE_GATE_UP, K_PRE_DOWN, K_COMBINE, K_CACHE_TABLE, K_PACK, K_ROUTE_PERMUTE, K_PRE_SPLIT,
    K_CACHE_MOVE, K_MICRO_READ, K_MICRO_MFMA, K_SCATTER, K_DEC_SMALL, K_COUNT
};

bool timing_enabled();
// When timing is enabled, hands out the two events a launch of kernel `kid`
// records its start and end in (they are read by moe_timing_query).
bool timing_begin(int kid, hipEvent_t *start, hipEvent_t *stop);

// Launch of kernel `kid`; with timing enabled the start and end of the
// dispatch itself land in two events on the launch stream (hipExtLaunchKernel).
#define MOE_LAUNCH(kid, kernel, grid, block, shmem, stream, ...)                              \
    do {                                                                                      \
        hipEvent_t moe_ev0_ = nullptr, moe_ev1_ = nullptr;                                    \
        if (::moe::timing_enabled() && ::moe::timing_begin((kid), &moe_ev0_, &moe_ev1_))      \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, moe_ev0_, moe_ev1_, 0,  \
                                  __VA_ARGS__);                                               \
        else                                                                                  \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);              \
    } while (0)

// ------------------------------------------------------------ bf16 bits --

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// Two fp32 -> two bf16 (lo in the low half), rounded to nearest even by the
// gfx950 packed convert (v_cvt_pk_bf16_f32; NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return pack_bf16x2(f, 0.0f) & 0xFFFFu;
}

// E8M0 scale byte -> fp32 multiplier 2^(s-127) (s = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
    return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}

// ------------------------------------------------------------- loads -----

// Loads through the global address space: pointers read from device tables
// are generic, and generic (FLAT) loads also count against the LDS/scalar
// wait counter, which would make every LDS wait also wait for them.
#define MOE_GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ u32x4 load_nt16(const void *p) {
    return __builtin_nontemporal_load((const MOE_GLOBAL u32x4 *)(p));
}

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *(const MOE_GLOBAL u32x4 *)(p);
}

__device__ __forceinline__ uint32_t load_u8(const void *p) {
    return *(const MOE_GLOBAL uint8_t *)(p);
}

__device__ __forceinline__ uint32_t load_u32(const void *p) {
    return *(const MOE_GLOBAL uint32_t *)(p);
}

// Raw buffer loads through a resource with a byte range: an offset at or past
// the range returns zeros without a memory access. A load that is issued on
// every path and switched off by its offset keeps the count of loads in
// flight the same on all paths, so the compiler's wait before a use can leave
// later loads (a prefetch) in flight instead of draining all of them where
// paths with and without the load merge.
using buf_rsrc = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kBufOff = 0x80000000u;   // past every range made here (< 2 GiB)
constexpr int kBufNt = 2;                    // non-temporal cache policy bit
__device__ __forceinline__ buf_rsrc make_rsrc(const void *base, uint32_t bytes) {
    // word 3 = 0x00020000: raw dword data format for the gfx9 family
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ u32x4 buf_load_nt16(buf_rsrc r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufNt);
}
__device__ __forceinline__ uint32_t buf_load_u8(buf_rsrc r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, kBufNt);
}

// Reads through the constant address space become scalar loads when the
// address is wavefront-uniform; they wait on the scalar counter and never on
// the vector loads in flight. Only for data the kernel does not write.
#define MOE_CONST __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ const MOE_CONST T *as_scalar(const T *p) {
    return (const MOE_CONST T *)(p);
}

#define MOE_LDS __attribute__((address_space(3)))

// Direct global -> LDS copies: lane l's 16 (4) bytes land at dst + 16 l (4 l);
// dst is wavefront-uniform.
__device__ __forceinline__ void lds_dma16(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds((const MOE_GLOBAL void *)src, (MOE_LDS void *)dst, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds((const MOE_GLOBAL void *)src, (MOE_LDS void *)dst, 4, 0, 0);
}

// Waits until at most n of this wavefront's vector-memory operations are
// outstanding (n < 64). gfx9 s_waitcnt fields: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt_hi[15:14].
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

// 8 MXFP4 codes (one dword, element 0 in the low nibble) -> 8 bf16 scaled by sc.
__device__ __forceinline__ bf16x8 dequant8_fp4(uint32_t w, float sc) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3);
    bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}

// ---------------------------------------------------------- wave utils ---

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l ? (~0ull >> (64 - l)) : 0ull;
}

// Index of the a-th (0-based) expert that received at least one pair, or -1.
// Called by a whole wavefront (all lanes get the same answer).
__device__ __forceinline__ int find_active_expert(const int32_t *__restrict__ offsets, int E, int a) {
    const int lane = lane_id();
    int seen = 0;
    for (int base = 0; base < E; base += kWave) {
        const int e = base + lane;
        const bool act = e < E && offsets[e + 1] > offsets[e];
        const uint64_t m = __ballot(act);
        const int c = __popcll(m);
        if (a < seen + c) {
            const int r = a - seen;
            const bool hit = act && __popcll(m & lanemask_lt()) == r;
            const uint64_t hm = __ballot(hit);
            return base + __ffsll((long long)hm) - 1;
        }
        seen += c;
    }
    return -1;
}

}  // namespace moe
