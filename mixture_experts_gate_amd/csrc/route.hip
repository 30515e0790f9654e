// Router: optional bf16 gate GEMV, top-k selection by wavefront arg-max, and
// renormalised softmax weights. One wavefront handles one token.
//
// The pages fix only that a few routed experts are active per token
// (winzheng.com page, "Why Now of All Times": six per layer); the selection
// rule (largest logits, ties to the lower index) and the renormalised
// softmax weights are the plain reading taken for the layer.
#include <math.h>

#include "common.hpp"

namespace moe {

// `a` (value av, index ai) ranks before `b`: larger logit, then lower index.
__device__ __forceinline__ bool ranks_before(float av, int ai, float bv, int bi) {
    return av > bv || (av == bv && ai < bi);
}

// Gate logit of token row x[H] against gate row w[H], in the fixed order:
// lane l sums (ascending h) the 8-element chunks c with c % 64 == l, then the
// lanes meet in a butterfly with distances 32..1. Every lane returns the sum.
__device__ __forceinline__ float gate_dot(const uint16_t *__restrict__ x,
                                          const uint16_t *__restrict__ w, int H) {
    const int lane = lane_id();
    float acc = 0.0f;
    for (int c = lane; c * 8 < H; c += kWave) {
        const u32x4 xv = load16(x + c * 8);
        const u32x4 wv = load16(w + c * 8);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            // products of bf16 pairs are exact in fp32, so fused or not gives the same sum
            acc += bf16_bits_to_f32(xv[q] & 0xFFFFu) * bf16_bits_to_f32(wv[q] & 0xFFFFu);
            acc += bf16_bits_to_f32(xv[q] >> 16) * bf16_bits_to_f32(wv[q] >> 16);
        }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d);
    return acc;
}

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg,
    const float *__restrict__ logits_in, float *__restrict__ logits_out, int T, int H, int E,
    int k, int renormalize, int32_t *__restrict__ topk_ids, float *__restrict__ topk_w) {
    const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    const int lane = lane_id();

    // logits of experts e = lane + 64*i
    float v[VPL];
    if (logits_in) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = lane + kWave * i;
            v[i] = e < E ? logits_in[(size_t)t * E + e] : 0.0f;
        }
    } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) v[i] = 0.0f;
        const uint16_t *xr = x + (size_t)t * H;
        for (int e = 0; e < E; ++e) {
            const float l = gate_dot(xr, wg + (size_t)e * H, H);
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (e == lane + kWave * i) v[i] = l;
        }
    }
    if (logits_out) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = lane + kWave * i;
            if (e < E) logits_out[(size_t)t * E + e] = v[i];
        }
    }

    // k rounds of wavefront arg-max over the not-yet-taken experts
    uint32_t taken = 0;
    float my_v = 0.0f, top_v = 0.0f;
    int my_i = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = lane + kWave * i;
            if (e < E && !((taken >> i) & 1u) && ranks_before(v[i], e, bv, bi)) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            const float ov = __shfl_xor(bv, d);
            const int oi = __shfl_xor(bi, d);
            if (ranks_before(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
        if (j == 0) top_v = bv;
        if (lane == j) {
            my_v = bv;
            my_i = bi;
        }
    }

    // weights: lanes j < k hold the j-th choice
    float num = lane < k ? expf(my_v - top_v) : 0.0f;
    float den;
    if (renormalize) {
        den = num;
    } else {
        den = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = lane + kWave * i;
            if (e < E) den += expf(v[i] - top_v);
        }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) den += __shfl_xor(den, d);
    if (lane < k) {
        topk_ids[(size_t)t * k + lane] = my_i;
        topk_w[(size_t)t * k + lane] = num / den;
    }
}

}  // namespace moe

using namespace moe;

extern "C" int moe_route(const uint16_t *x_bf16, const uint16_t *wg_bf16, const float *logits_in,
                         float *logits_out, int T, int H, int E, int k, int renormalize,
                         int32_t *topk_ids, float *topk_w, void *stream) {
    if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > kWave) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!topk_ids || !topk_w) return MOE_EINVAL;
    if (!logits_in) {
        if (!x_bf16 || !wg_bf16 || H < 8 || H % 8) return MOE_EINVAL;
    }
    hipStream_t s = (hipStream_t)stream;
    const int waves_per_block = 4;
    dim3 grid((T + waves_per_block - 1) / waves_per_block), block(kWave * waves_per_block);
#define MOE_ROUTE_LAUNCH(VPL)                                                                 \
    MOE_TIMED(s, K_ROUTE,                                                                     \
              hipLaunchKernelGGL(route_kernel<VPL>, grid, block, 0, s, x_bf16, wg_bf16,       \
                                 logits_in, logits_out, T, H, E, k, renormalize, topk_ids,    \
                                 topk_w))
    if (E <= 64) MOE_ROUTE_LAUNCH(1);
    else if (E <= 128) MOE_ROUTE_LAUNCH(2);
    else if (E <= 256) MOE_ROUTE_LAUNCH(4);
    else if (E <= 512) MOE_ROUTE_LAUNCH(8);
    else MOE_ROUTE_LAUNCH(16);
#undef MOE_ROUTE_LAUNCH
    return check_launch();
}
