// Device code of the router (one wavefront per token), shared by the router
// kernel and the fused router + permutation kernel.
//
// The pages fix only that a few routed experts are active per token
// (winzheng.com page, "Why Now of All Times": six per layer); the selection
// rule (largest logits, ties to the lower index) and the renormalised
// softmax weights are the plain reading taken for the layer.
#pragma once
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

// ---- wavefront reductions with DPP (rows of 16) and lane reads (across rows)

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
    return (uint64_t)dpp32<CTRL>((uint32_t)v) | ((uint64_t)dpp32<CTRL>((uint32_t)(v >> 32)) << 32);
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
    return (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l) |
           ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l) << 32);
}

// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror:4, row_ror:8
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRor4 = 0x124, kDppRor8 = 0x128;

// DPP move of a 64-bit value restricted to the rows in ROWS (other rows get 0,
// which ranks last).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp64_rows(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWS, 0xF, false);
    return (uint64_t)lo | ((uint64_t)hi << 32);
}

// DPP controls: row_bcast:15 (lane 15 of each row into the next row),
// row_bcast:31 (lane 31 into rows 2 and 3)
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;

// Maximum of a 64-bit key over the wavefront (wavefront-uniform result). The
// whole reduction stays in the vector unit (the row maxima meet in lane 63 by
// row broadcasts) and one lane read hands the result out: lane reads of each
// row's maximum followed by scalar comparisons cost a round trip between the
// vector and scalar units per step.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
    k = max_u64(k, dpp64<kDppXor1>(k));
    k = max_u64(k, dpp64<kDppXor2>(k));
    k = max_u64(k, dpp64<kDppRor4>(k));
    k = max_u64(k, dpp64<kDppRor8>(k));
    k = max_u64(k, dpp64_rows<kDppBcast15, 0xA>(k));
    k = max_u64(k, dpp64_rows<kDppBcast31, 0xC>(k));
    return readlane64(k, kWave - 1);
}

// Sum over the wavefront in a fixed order (wavefront-uniform result).
__device__ __forceinline__ float wave_sum(float v) {
    v += __uint_as_float(dpp32<kDppXor1>(__float_as_uint(v)));
    v += __uint_as_float(dpp32<kDppXor2>(__float_as_uint(v)));
    v += __uint_as_float(dpp32<kDppRor4>(__float_as_uint(v)));
    v += __uint_as_float(dpp32<kDppRor8>(__float_as_uint(v)));
    return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48)));
}

// Total order "ranks before" as an unsigned key: larger logit first, then
// lower expert index. -0.0 is folded into +0.0 first (they compare equal).
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
    const uint32_t u = __float_as_uint(v + 0.0f);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ __forceinline__ float key_value(uint64_t key) {
    const uint32_t ord = (uint32_t)(key >> 32);
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

__device__ __forceinline__ int key_index(uint64_t key) { return (int)(~(uint32_t)key); }

// Logits of token t held as v[i] = logit of expert lane + 64 i (from logits_in,
// or from the gate when logits_in is NULL).
template <int VPL>
__device__ __forceinline__ void token_logits(int t, const uint16_t *__restrict__ x,
                                             const uint16_t *__restrict__ wg,
                                             const float *__restrict__ logits_in, int H, int E,
                                             float (&v)[VPL]) {
    const int lane = lane_id();
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
}

// Routes TB tokens t0 + b * tstride (b < TB, those below T) with one
// wavefront from their logits v[b]: k rounds of arg-max (the TB tokens'
// rounds are independent and interleave), then the weights. Lanes j < k write
// choice j of each token; id[b] receives the lane's expert id (-1 for lanes >= k).
template <int VPL, int TB>
__device__ __forceinline__ void route_from_logits(int t0, int tstride, int T,
                                                  const float (&v)[TB][VPL],
                                                  float *__restrict__ logits_out, int E, int k,
                                                  int renormalize, int32_t *__restrict__ topk_ids,
                                                  float *__restrict__ topk_w, int (&id)[TB]) {
    const int lane = lane_id();
    uint64_t key[TB][VPL];
    float my_v[TB], top_v[TB];
    int my_i[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
        const int t = t0 + b * tstride;
        my_v[b] = top_v[b] = 0.0f;
        my_i[b] = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int e = lane + kWave * i;
            key[b][i] = (t < T && e < E) ? rank_key(v[b][i], e) : 0ull;  // 0 ranks last
            if (logits_out && t < T && e < E) logits_out[(size_t)t * E + e] = v[b][i];
        }
    }
    for (int j = 0; j < k; ++j) {
#pragma unroll
        for (int b = 0; b < TB; ++b) {
            uint64_t best = 0;
#pragma unroll
            for (int i = 0; i < VPL; ++i) best = max_u64(best, key[b][i]);
            const uint64_t win = wave_max_u64(best);
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                if (key[b][i] == win) key[b][i] = 0;            // taken
            const float wv = key_value(win);
            if (j == 0) top_v[b] = wv;
            if (lane == j) {
                my_v[b] = wv;
                my_i[b] = key_index(win);
            }
        }
    }
#pragma unroll
    for (int b = 0; b < TB; ++b) {
        const int t = t0 + b * tstride;
        id[b] = -1;
        if (t >= T) continue;
        // weights: lanes j < k hold the j-th choice
        const float num = lane < k ? expf(my_v[b] - top_v[b]) : 0.0f;
        float den;
        if (renormalize) {
            den = wave_sum(num);
        } else {
            float part = 0.0f;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                const int e = lane + kWave * i;
                if (e < E) part += expf(v[b][i] - top_v[b]);
            }
            den = wave_sum(part);
        }
        if (lane < k) {
            topk_ids[(size_t)t * k + lane] = my_i[b];
            topk_w[(size_t)t * k + lane] = num / den;
            id[b] = my_i[b];
        }
    }
}

template <int VPL>
__device__ __forceinline__ int route_token(int t, const uint16_t *__restrict__ x,
                                           const uint16_t *__restrict__ wg,
                                           const float *__restrict__ logits_in,
                                           float *__restrict__ logits_out, int H, int E, int k,
                                           int renormalize, int32_t *__restrict__ topk_ids,
                                           float *__restrict__ topk_w) {
    float v[1][VPL];
    token_logits<VPL>(t, x, wg, logits_in, H, E, v[0]);
    int id[1];
    route_from_logits<VPL, 1>(t, 0, t + 1, v, logits_out, E, k, renormalize, topk_ids, topk_w, id);
    return id[0];
}

}  // namespace moe
