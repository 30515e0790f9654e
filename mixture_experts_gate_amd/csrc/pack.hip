// Interchange (row-major) MXFP4 -> kernel layout (16-row x 128-column blocks
// stored contiguously in matrix-core lane order). One thread moves the 16
// code bytes and the scale byte that one lane of a decode wavefront reads.
#include "common.hpp"

namespace moe {

// One matrix of R rows x K columns; blocks (rb, s) of 64 lanes each.
__global__ __launch_bounds__(256) void pack_mxfp4_kernel(const uint8_t *__restrict__ src_base,
                                                         uint8_t *__restrict__ dst_base,
                                                         size_t src_stride, size_t dst_stride,
                                                         size_t o_codes, size_t o_scales, int R,
                                                         int K) {
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
    const u32x4 v = load16(src + o_codes + row * (K / 2) + (size_t)cb * 16);
    *reinterpret_cast<u32x4 *>(dst + o_codes + (size_t)blk * 1024 + l * 16) = v;
    dst[o_scales + (size_t)blk * 64 + l] = src[o_scales + row * (K / 32) + cb];
}

}  // namespace moe

using namespace moe;

extern "C" int moe_pack_mxfp4(const void *src, void *dst, int n, size_t src_stride,
                              size_t dst_stride, int H, int I, size_t lay_w13, size_t lay_s13,
                              size_t lay_w2, size_t lay_s2, void *stream) {
    if (n < 0 || H < 128 || I < 128 || H % 128 || I % 128) return MOE_EINVAL;
    if (n == 0) return MOE_OK;
    if (!src || !dst || n > 65535) return MOE_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    const uint8_t *sp = reinterpret_cast<const uint8_t *>(src);
    uint8_t *dp = reinterpret_cast<uint8_t *>(dst);
    // W13: 2I rows x H columns; W2: H rows x I columns
    const long l13 = (long)(2 * I / 16) * (H / 128) * 64;
    const long l2 = (long)(H / 16) * (I / 128) * 64;
    MOE_LAUNCH(K_PACK, pack_mxfp4_kernel, dim3((unsigned)((l13 + 255) / 256), n),
                                 dim3(256), 0, s, sp, dp, src_stride, dst_stride, lay_w13, lay_s13,
                                 2 * I, H);
    int rc = check_launch();
    if (rc) return rc;
    MOE_LAUNCH(K_PACK, pack_mxfp4_kernel, dim3((unsigned)((l2 + 255) / 256), n),
                                 dim3(256), 0, s, sp, dp, src_stride, dst_stride, lay_w2, lay_s2,
                                 H, I);
    return check_launch();
}
