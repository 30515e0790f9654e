// Interchange (row-major) -> kernel layout of block-scaled and FP8 expert
// weights: 16-row x 128-column blocks stored contiguously in matrix-core lane
// order. One thread moves what one lane of a decode wavefront reads for one
// block: MXFP4 16 code bytes + 1 scale byte, NVFP4 16 code bytes + 2 scale
// bytes, FP8 32 code bytes. Per-matrix fp32 scales (NVFP4, FP8) are copied as
// they are.
#include "common.hpp"

namespace moe {

// One matrix of R rows x K columns; blocks (rb, s) of 64 lanes each.
template <int FMT>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t *__restrict__ src_base,
                                                   uint8_t *__restrict__ dst_base,
                                                   size_t src_stride, size_t dst_stride,
                                                   size_t o_codes, size_t o_scales, int R, int K) {
    const int nslab = K / 128;
    const long lanes = (long)(R / 16) * nslab * 64;
    const long g = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= lanes) return;
    const uint8_t *src = src_base + (size_t)blockIdx.y * src_stride;
    uint8_t *dst = dst_base + (size_t)blockIdx.y * dst_stride;
    const int l = (int)(g & 63);
    const long blk = g >> 6;                 // rb * nslab + s
    const int rb = (int)(blk / nslab), s = (int)(blk - (long)rb * nslab);
    const long row = (long)rb * 16 + (l & 15);
    const int cb = s * 4 + (l >> 4);         // 32-column block index
    if (FMT == MOE_W_FP8) {
        const uint8_t *sp = src + o_codes + row * K + (size_t)cb * 32;
        uint8_t *dp = dst + o_codes + (size_t)blk * 2048 + l * 32;
        *reinterpret_cast<u32x4 *>(dp) = load16(sp);
        *reinterpret_cast<u32x4 *>(dp + 16) = load16(sp + 16);
        if (g == 0)     // the matrix's fp32 scale (16-byte field)
            *reinterpret_cast<u32x4 *>(dst + o_scales) = load16(src + o_scales);
        return;
    }
    const u32x4 v = load16(src + o_codes + row * (K / 2) + (size_t)cb * 16);
    *reinterpret_cast<u32x4 *>(dst + o_codes + (size_t)blk * 1024 + l * 16) = v;
    if (FMT == MOE_W_MXFP4) {
        dst[o_scales + (size_t)blk * 64 + l] = src[o_scales + row * (K / 32) + cb];
    } else {
        const size_t si = o_scales + row * (K / 16) + (size_t)cb * 2;
        dst[o_scales + (size_t)blk * 128 + l * 2] = src[si];
        dst[o_scales + (size_t)blk * 128 + l * 2 + 1] = src[si + 1];
        if (g == 0) {   // the matrix's fp32 scale after the block scales
            const size_t o = o_scales + (size_t)R * (K / 16);
            *reinterpret_cast<u32x4 *>(dst + o) = load16(src + o);
        }
    }
}

template <int FMT>
static int pack_fmt(const uint8_t *sp, uint8_t *dp, int n, size_t src_stride, size_t dst_stride,
                    int H, int I, size_t lay_w13, size_t lay_s13, size_t lay_w2, size_t lay_s2,
                    hipStream_t s) {
    // W13: 2I rows x H columns; W2: H rows x I columns
    const long l13 = (long)(2 * I / 16) * (H / 128) * 64;
    const long l2 = (long)(H / 16) * (I / 128) * 64;
    MOE_LAUNCH(K_PACK, pack_kernel<FMT>, dim3((unsigned)((l13 + 255) / 256), n), dim3(256), 0, s,
               sp, dp, src_stride, dst_stride, lay_w13, lay_s13, 2 * I, H);
    int rc = check_launch();
    if (rc) return rc;
    MOE_LAUNCH(K_PACK, pack_kernel<FMT>, dim3((unsigned)((l2 + 255) / 256), n), dim3(256), 0, s,
               sp, dp, src_stride, dst_stride, lay_w2, lay_s2, H, I);
    return check_launch();
}

}  // namespace moe

using namespace moe;

extern "C" int moe_pack_weights(int fmt, const void *src, void *dst, int n, size_t src_stride,
                                size_t dst_stride, int H, int I, size_t lay_w13, size_t lay_s13,
                                size_t lay_w2, size_t lay_s2, void *stream) {
    if (fmt != MOE_W_MXFP4 && fmt != MOE_W_NVFP4 && fmt != MOE_W_FP8) return MOE_EINVAL;
    if (n < 0 || H < 128 || I < 128 || H % 128 || I % 128) return MOE_EINVAL;
    if (n == 0) return MOE_OK;
    if (!src || !dst || n > 65535) return MOE_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    const uint8_t *sp = reinterpret_cast<const uint8_t *>(src);
    uint8_t *dp = reinterpret_cast<uint8_t *>(dst);
    if (fmt == MOE_W_MXFP4)
        return pack_fmt<MOE_W_MXFP4>(sp, dp, n, src_stride, dst_stride, H, I, lay_w13, lay_s13,
                                     lay_w2, lay_s2, s);
    if (fmt == MOE_W_NVFP4)
        return pack_fmt<MOE_W_NVFP4>(sp, dp, n, src_stride, dst_stride, H, I, lay_w13, lay_s13,
                                     lay_w2, lay_s2, s);
    return pack_fmt<MOE_W_FP8>(sp, dp, n, src_stride, dst_stride, H, I, lay_w13, lay_s13, lay_w2,
                               lay_s2, s);
}

extern "C" int moe_pack_mxfp4(const void *src, void *dst, int n, size_t src_stride,
                              size_t dst_stride, int H, int I, size_t lay_w13, size_t lay_s13,
                              size_t lay_w2, size_t lay_s2, void *stream) {
    return moe_pack_weights(MOE_W_MXFP4, src, dst, n, src_stride, dst_stride, H, I, lay_w13,
                            lay_s13, lay_w2, lay_s2, stream);
}
