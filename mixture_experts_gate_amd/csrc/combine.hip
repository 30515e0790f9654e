// Weighted combine of each token's k expert outputs (plus the always-on
// shared expert when given). Memory-bound: each thread owns 8 consecutive
// hidden elements of one token and sums its k rows in fp32, j ascending.
#include "common.hpp"

namespace moe {

template <bool YF32>
__device__ __forceinline__ void load8(const void *base, size_t off, float v[8]) {
    if (YF32) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(base) + off);
        const f32x4 b =
            *reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(base) + off + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = a[i];
            v[4 + i] = b[i];
        }
    } else {
        const u32x4 q = load16(reinterpret_cast<const uint16_t *>(base) + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_bits_to_f32(q[i] & 0xFFFFu);
            v[2 * i + 1] = bf16_bits_to_f32(q[i] >> 16);
        }
    }
}

// KMAX > 0: k == KMAX known at compile time (all k row loads issued at once).
template <bool YF32, int KMAX>
__global__ __launch_bounds__(64) void combine_kernel(const void *__restrict__ y,
                                                     const float *__restrict__ w,
                                                     const void *__restrict__ ysh, int T, int k,
                                                     int H, uint16_t *__restrict__ out) {
    const int per_tok = H / 8;
    const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (long)T * per_tok) return;
    const int t = (int)(gid / per_tok), h8 = (int)(gid - (long)t * per_tok) * 8;
    const int kk = KMAX > 0 ? KMAX : k;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (KMAX > 0) {
        float v[KMAX > 0 ? KMAX : 1][8];
        float wj[KMAX > 0 ? KMAX : 1];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            wj[j] = w[(size_t)t * KMAX + j];
            load8<YF32>(y, ((size_t)t * KMAX + j) * H + h8, v[j]);
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += wj[j] * v[j][i];
    } else {
        for (int j = 0; j < kk; ++j) {
            const float wj = w[(size_t)t * kk + j];
            float v[8];
            load8<YF32>(y, ((size_t)t * kk + j) * H + h8, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += wj * v[i];
        }
    }
    if (ysh) {
        float v[8];
        load8<YF32>(ysh, (size_t)t * H + h8, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *reinterpret_cast<u32x4 *>(out + (size_t)t * H + h8) = o;
}

template <bool YF32>
static void launch_combine(dim3 grid, hipStream_t s, const void *y, const float *w, const void *ysh,
                           int T, int k, int H, uint16_t *out) {
#define MOE_CB(KM)                                                                            \
    MOE_LAUNCH(K_COMBINE, (combine_kernel<YF32, KM>), grid, dim3(64), 0, s, y, w, ysh, T, \
                                 k, H, out)
    switch (k) {
        case 1: MOE_CB(1); break;
        case 2: MOE_CB(2); break;
        case 4: MOE_CB(4); break;
        case 6: MOE_CB(6); break;
        case 8: MOE_CB(8); break;
        default: MOE_CB(0); break;
    }
#undef MOE_CB
}

// dst row idx[r] = src row r, rows of row_bytes bytes (a multiple of 16): one
// workgroup per row.
__global__ __launch_bounds__(256) void scatter_rows_kernel(const u32x4 *__restrict__ src,
                                                           const int32_t *__restrict__ idx,
                                                           size_t row16, u32x4 *__restrict__ dst) {
    const int r = blockIdx.x;
    const size_t to = (size_t)idx[r];
    for (size_t i = threadIdx.x; i < row16; i += blockDim.x)
        dst[to * row16 + i] = src[(size_t)r * row16 + i];
}

}  // namespace moe

using namespace moe;

extern "C" int moe_scatter_rows(const void *src, const int32_t *idx, int n, size_t row_bytes,
                                void *dst, void *stream) {
    if (n < 0 || row_bytes == 0 || row_bytes % 16) return MOE_EINVAL;
    if (n == 0) return MOE_OK;
    if (!src || !idx || !dst) return MOE_EINVAL;
    MOE_LAUNCH(K_SCATTER, scatter_rows_kernel, dim3((unsigned)n), dim3(256), 0,
               (hipStream_t)stream, reinterpret_cast<const u32x4 *>(src), idx, row_bytes / 16,
               reinterpret_cast<u32x4 *>(dst));
    return check_launch();
}

extern "C" int moe_combine(const void *y, int y_is_fp32, const float *topk_w, const void *y_shared,
                           int T, int k, int H, uint16_t *out_bf16, void *stream) {
    if (T < 0 || k < 1 || H < 8 || H % 8) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!y || !topk_w || !out_bf16) return MOE_EINVAL;
    const long n = (long)T * (H / 8);
    dim3 grid((unsigned)((n + 63) / 64));
    hipStream_t s = (hipStream_t)stream;
    if (y_is_fp32) launch_combine<true>(grid, s, y, topk_w, y_shared, T, k, H, out_bf16);
    else launch_combine<false>(grid, s, y, topk_w, y_shared, T, k, H, out_bf16);
    return check_launch();
}
