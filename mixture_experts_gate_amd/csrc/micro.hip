// Measurement kernels for the rooflines the layer's kernels are judged
// against: a read stream over a device buffer (HBM bytes per second at a
// given size and launch shape) and matrix-core issue loops (FLOPs per second
// of the bf16 and the block-scaled FP8 x FP4 instructions the layer uses).
// They compute nothing of the layer.
#include "common.hpp"

namespace moe {

typedef __attribute__((ext_vector_type(8))) int i32x8;
constexpr uint32_t kSinkMagic = 0x9E3779B9u;   // written only if a result equals it

// Workgroups take 64 KB chunks of the buffer in turn (chunk c goes to
// workgroup c mod grid); each lane keeps 16 non-temporal 16-byte loads of a
// chunk in flight. The XOR of everything read is kept live by a store that
// happens only if it equals a constant.
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4 *__restrict__ buf,
                                                          size_t n16, uint32_t *sink) {
    constexpr size_t kChunk16 = 4096;   // 16-byte units per chunk
    uint32_t acc = 0;
    for (size_t c = blockIdx.x; c * kChunk16 < n16; c += gridDim.x) {
        const size_t base = c * kChunk16 + threadIdx.x;
        u32x4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const size_t i = base + (size_t)u * 256;
            v[u] = i < n16 ? load_nt16(buf + i) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == kSinkMagic) sink[0] = acc;
}

// KIND 0: v_mfma_f32_32x32x16_bf16 (32768 FLOPs each); KIND 1:
// v_mfma_scale_f32_16x16x128_f8f6f4 with an E2M1 A operand and an E4M3 B
// operand (65536 FLOPs each). Four independent accumulator chains per wave.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, uint32_t *sink) {
    const int l = threadIdx.x;
    float out = 0.0f;
    if constexpr (KIND == 0) {
        bf16x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = (__bf16)(float)((l + i) & 7);
            b[i] = (__bf16)(float)((l * 3 + i) & 7);
        }
        f32x16 c[4] = {};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) out += c[j][i];
    } else {
        i32x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[i] = 0x22222222 + l + i;
            b[i] = 0x38383838 + l * 3 + i;
        }
        f32x4 c[4] = {};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[j], 4, 0, 0, 127, 0,
                                                                        127);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) out += c[j][i];
    }
    if (__float_as_uint(out) == kSinkMagic) sink[0] = __float_as_uint(out);
}

}  // namespace moe

using namespace moe;

extern "C" int moe_micro_read(const void *buf, size_t bytes, int grid, void *sink, void *stream) {
    if (!buf || !sink || grid < 1 || bytes < 16 || bytes % 16 ||
        reinterpret_cast<uintptr_t>(buf) % 16)
        return MOE_EINVAL;
    MOE_LAUNCH(K_MICRO_READ, read_stream_kernel, dim3((unsigned)grid), dim3(256), 0,
               (hipStream_t)stream, reinterpret_cast<const u32x4 *>(buf), bytes / 16,
               reinterpret_cast<uint32_t *>(sink));
    return check_launch();
}

extern "C" int moe_micro_mfma(int kind, int grid, int iters, void *sink, double *flops,
                              void *stream) {
    if ((kind != 0 && kind != 1) || grid < 1 || iters < 1 || !sink) return MOE_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (kind == 0)
        MOE_LAUNCH(K_MICRO_MFMA, mfma_loop_kernel<0>, dim3((unsigned)grid), dim3(256), 0, s, iters,
                   reinterpret_cast<uint32_t *>(sink));
    else
        MOE_LAUNCH(K_MICRO_MFMA, mfma_loop_kernel<1>, dim3((unsigned)grid), dim3(256), 0, s, iters,
                   reinterpret_cast<uint32_t *>(sink));
    // 4 waves per workgroup, 4 chains per wave
    if (flops) *flops = (double)grid * 4 * 4 * iters * (kind == 0 ? 32768.0 : 65536.0);
    return check_launch();
}
