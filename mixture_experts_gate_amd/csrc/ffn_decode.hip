// Decode-shaped grouped SwiGLU expert FFN: few tokens per expert, so the cost
// is streaming each touched expert's weights once from HBM.
//
// The pages place the cost of decoding a sparse MoE in expert-weight movement
// (winzheng.com page, "Why Now of All Times": only the routed experts'
// parameters take part per token). Here every touched expert's weights are
// read exactly once, coalesced and non-temporal, decoded in registers
// (E2M1 x E8M0 -> bf16 with the gfx950 scaled convert) and fed to bf16
// matrix-core instructions whose other operand is the expert's tokens.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 as used here: lane l supplies row
// (l % 16) and K-chunk (l / 16) of A (8 consecutive K), column (l % 16) and
// the same K-chunk of B; it receives D[4 * (l / 16) + i][l % 16], i = 0..3.
// A lane loads 16 bytes = 32 FP4 weights = one scale block; its 4 groups of 8
// feed 4 MFMAs, and the token operand is loaded with the same K mapping, so
// the K order inside an MFMA is a consistent permutation on both sides.
//
// Kernel 1 (gate/up + SwiGLU): one workgroup = 16 gate rows + the matching 16
// up rows of one touched expert; its 4 wavefronts split K and meet in LDS.
// Kernel 2 (down): one workgroup = 64 output rows (16 per wavefront) of one
// touched expert, full K per wavefront.
// Both grids are fixed by (min(E, T*k) touched-expert slots) x (row groups);
// each workgroup finds its expert from the device offsets, so nothing depends
// on a host round trip.
#include <math.h>

#include "common.hpp"

namespace moe {

constexpr int kTokPerPass = 64;     // tokens (4 groups of 16) per weight pass
constexpr int kGroups = kTokPerPass / 16;

__device__ __forceinline__ float silu_mul(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

// Weight fragment of one lane for one 32-element K block: 4 x bf16x8.
template <int FMT>
struct WFrag;

template <>
struct WFrag<MOE_W_MXFP4> {
    u32x4 q;
    uint32_t s;
    __device__ __forceinline__ void load(const uint8_t *codes_row, const uint8_t *scales_row,
                                         int kb, bool ok) {
        if (ok) {
            q = load_nt16(codes_row + (size_t)kb * 16);
            s = scales_row[kb];
        } else {
            q = u32x4{0, 0, 0, 0};
            s = 127;
        }
    }
    __device__ __forceinline__ bf16x8 get(int j) const { return dequant8_fp4(q[j], e8m0_to_f32(s)); }
};

template <>
struct WFrag<MOE_W_BF16> {
    u32x4 q[4];
    __device__ __forceinline__ void load(const uint8_t *row, const uint8_t *, int kb, bool ok) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            q[j] = ok ? load_nt16(row + (size_t)kb * 64 + j * 16) : u32x4{0, 0, 0, 0};
    }
    __device__ __forceinline__ bf16x8 get(int j) const { return as_bf16x8(q[j]); }
};

// Byte address of row `r` of a weight matrix with K columns.
template <int FMT>
__device__ __forceinline__ const uint8_t *wrow(const void *base, long r, int K) {
    return reinterpret_cast<const uint8_t *>(base) + (FMT == MOE_W_MXFP4 ? r * (K / 2) : r * K * 2);
}

__device__ __forceinline__ const uint8_t *srow(const uint8_t *base, long r, int K) {
    return base ? base + r * (K / 32) : nullptr;
}

// -------------------------------------------------------------- kernel 1 --
// SPW: 128-wide K slabs per wavefront (4 wavefronts cover ceil(H/128) slabs).
template <int FMT, int SPW>
__global__ __launch_bounds__(256) void ffn_dec_gate_up(
    const uint16_t *__restrict__ x, const int32_t *__restrict__ sorted_pair,
    const int32_t *__restrict__ offsets, const moe_expert_w *__restrict__ experts, int k, int H,
    int I, int E, uint16_t *__restrict__ act) {
    __shared__ float red[3][kGroups][2][4][kWave];
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    const int nrg = I / 16;
    const int a = blockIdx.x / nrg, rg = blockIdx.x - a * nrg;
    const int e = find_active_expert(offsets, E, a);
    if (e < 0) return;
    const int row0 = offsets[e], n_e = offsets[e + 1] - row0;
    const moe_expert_w W = experts[e];
    const int m = lane & 15, c = lane >> 4;
    const int nblk = H / 32;

    const uint8_t *rg_codes = wrow<FMT>(W.w13, rg * 16 + m, H);
    const uint8_t *ru_codes = wrow<FMT>(W.w13, I + rg * 16 + m, H);
    const uint8_t *rg_sc = srow(W.s13, rg * 16 + m, H);
    const uint8_t *ru_sc = srow(W.s13, I + rg * 16 + m, H);

    WFrag<FMT> fg[SPW], fu[SPW];
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int kb = (wv * SPW + i) * 4 + c;
        fg[i].load(rg_codes, rg_sc, kb, kb < nblk);
        fu[i].load(ru_codes, ru_sc, kb, kb < nblk);
    }

    for (int g0 = 0; g0 < n_e; g0 += kTokPerPass) {
        f32x4 accg[kGroups], accu[kGroups];
        const uint16_t *xrow[kGroups];
        bool has[kGroups];
#pragma unroll
        for (int gi = 0; gi < kGroups; ++gi) {
            accg[gi] = f32x4{0, 0, 0, 0};
            accu[gi] = f32x4{0, 0, 0, 0};
            const int r = g0 + gi * 16 + m;
            has[gi] = r < n_e;
            xrow[gi] = x + (size_t)(has[gi] ? sorted_pair[row0 + r] / k : 0) * H;
        }
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int kb = (wv * SPW + i) * 4 + c;
            bf16x8 ag[4], au[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ag[j] = fg[i].get(j);
                au[j] = fu[i].get(j);
            }
#pragma unroll
            for (int gi = 0; gi < kGroups; ++gi) {
                if (g0 + gi * 16 >= n_e) break;      // wavefront-uniform
                const bool ld = has[gi] && kb < nblk;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8 b =
                        ld ? as_bf16x8(load16(xrow[gi] + kb * 32 + j * 8)) : bf16x8{};
                    accg[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag[j], b, accg[gi], 0, 0, 0);
                    accu[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au[j], b, accu[gi], 0, 0, 0);
                }
            }
        }
        // K-split partial sums meet in LDS; wavefront 0 adds them in order 0,1,2,3
        if (wv > 0) {
#pragma unroll
            for (int gi = 0; gi < kGroups; ++gi) {
                if (g0 + gi * 16 >= n_e) break;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    red[wv - 1][gi][0][i][lane] = accg[gi][i];
                    red[wv - 1][gi][1][i][lane] = accu[gi][i];
                }
            }
        }
        __syncthreads();
        if (wv == 0) {
#pragma unroll
            for (int gi = 0; gi < kGroups; ++gi) {
                if (g0 + gi * 16 >= n_e) break;
                const int r = g0 + gi * 16 + m;
                float o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float gs = accg[gi][i], us = accu[gi][i];
#pragma unroll
                    for (int w = 0; w < 3; ++w) {
                        gs += red[w][gi][0][i][lane];
                        us += red[w][gi][1][i][lane];
                    }
                    o[i] = silu_mul(gs, us);
                }
                if (r < n_e) {
                    uint2 pk;
                    pk.x = pack_bf16x2(o[0], o[1]);
                    pk.y = pack_bf16x2(o[2], o[3]);
                    *reinterpret_cast<uint2 *>(act + (size_t)(row0 + r) * I + rg * 16 + 4 * c) = pk;
                }
            }
        }
        __syncthreads();
    }
}

// -------------------------------------------------------------- kernel 2 --
// SPK: 128-wide K slabs (K = I) per wavefront, covering all of I.
template <int FMT, int SPK, bool YF32>
__global__ __launch_bounds__(256) void ffn_dec_down(
    const uint16_t *__restrict__ act, const int32_t *__restrict__ sorted_pair,
    const int32_t *__restrict__ offsets, const moe_expert_w *__restrict__ experts, int H, int I,
    int E, void *__restrict__ y) {
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    const int ncg = (H + 63) / 64;
    const int a = blockIdx.x / ncg, cg = blockIdx.x - a * ncg;
    const int e = find_active_expert(offsets, E, a);
    if (e < 0) return;
    const int nbase = cg * 64 + wv * 16;
    if (nbase >= H) return;
    const int row0 = offsets[e], n_e = offsets[e + 1] - row0;
    const moe_expert_w W = experts[e];
    const int m = lane & 15, c = lane >> 4;
    const int nblk = I / 32;

    const uint8_t *codes = wrow<FMT>(W.w2, nbase + m, I);
    const uint8_t *sc = srow(W.s2, nbase + m, I);
    WFrag<FMT> f[SPK];
#pragma unroll
    for (int i = 0; i < SPK; ++i) {
        const int kb = i * 4 + c;
        f[i].load(codes, sc, kb, kb < nblk);
    }

    for (int g0 = 0; g0 < n_e; g0 += kTokPerPass) {
        f32x4 acc[kGroups];
        bool has[kGroups];
#pragma unroll
        for (int gi = 0; gi < kGroups; ++gi) {
            acc[gi] = f32x4{0, 0, 0, 0};
            has[gi] = g0 + gi * 16 + m < n_e;
        }
#pragma unroll
        for (int i = 0; i < SPK; ++i) {
            const int kb = i * 4 + c;
            bf16x8 w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = f[i].get(j);
#pragma unroll
            for (int gi = 0; gi < kGroups; ++gi) {
                if (g0 + gi * 16 >= n_e) break;
                const bool ld = has[gi] && kb < nblk;
                const uint16_t *arow = act + (size_t)(row0 + g0 + gi * 16 + m) * I + kb * 32;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8 b = ld ? as_bf16x8(load16(arow + j * 8)) : bf16x8{};
                    acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[j], b, acc[gi], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int gi = 0; gi < kGroups; ++gi) {
            if (g0 + gi * 16 >= n_e) break;
            if (!has[gi]) continue;
            const int p = sorted_pair[row0 + g0 + gi * 16 + m];
            const size_t off = (size_t)p * H + nbase + 4 * c;
            if (YF32) {
                *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(y) + off) = acc[gi];
            } else {
                uint2 pk;
                pk.x = pack_bf16x2(acc[gi][0], acc[gi][1]);
                pk.y = pack_bf16x2(acc[gi][2], acc[gi][3]);
                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(y) + off) = pk;
            }
        }
    }
}

// ------------------------------------------------------------- launchers --

template <int FMT>
static int launch_gate_up(int spw, dim3 grid, hipStream_t s, const uint16_t *x, const int32_t *sp,
                          const int32_t *off, const moe_expert_w *ex, int k, int H, int I, int E,
                          uint16_t *act) {
#define MOE_GU(N)                                                                          \
    MOE_TIMED(s, K_DEC_GATE_UP,                                                            \
              hipLaunchKernelGGL((ffn_dec_gate_up<FMT, N>), grid, dim3(256), 0, s, x, sp, off, \
                                 ex, k, H, I, E, act))
    switch (spw) {
        case 1: MOE_GU(1); break;
        case 2: MOE_GU(2); break;
        case 4: MOE_GU(4); break;
        case 8: MOE_GU(8); break;
        default: return MOE_EUNSUPPORTED;
    }
#undef MOE_GU
    return check_launch();
}

template <int FMT, bool YF32>
static int launch_down(int spk, dim3 grid, hipStream_t s, const uint16_t *act, const int32_t *sp,
                       const int32_t *off, const moe_expert_w *ex, int H, int I, int E, void *y) {
#define MOE_DN(N)                                                                             \
    MOE_TIMED(s, K_DEC_DOWN,                                                                  \
              hipLaunchKernelGGL((ffn_dec_down<FMT, N, YF32>), grid, dim3(256), 0, s, act, sp, \
                                 off, ex, H, I, E, y))
    switch (spk) {
        case 2: MOE_DN(2); break;
        case 4: MOE_DN(4); break;
        case 6: MOE_DN(6); break;
        case 8: MOE_DN(8); break;
        case 16: MOE_DN(16); break;
        default: return MOE_EUNSUPPORTED;
    }
#undef MOE_DN
    return check_launch();
}

static int round_slabs(int slabs, const int *choices, int n) {
    for (int i = 0; i < n; ++i)
        if (slabs <= choices[i]) return choices[i];
    return -1;
}

int ffn_decode(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
               const moe_expert_w *experts, int fmt, int T, int k, int H, int I, int E, void *y,
               int y_is_fp32, uint16_t *act, hipStream_t s) {
    const int slabs_h = (H + 127) / 128, slabs_i = (I + 127) / 128;
    static const int spw_choices[] = {1, 2, 4, 8};
    static const int spk_choices[] = {2, 4, 6, 8, 16};
    const int spw = round_slabs((slabs_h + 3) / 4, spw_choices, 4);
    const int spk = round_slabs(slabs_i, spk_choices, 5);
    if (spw < 0 || spk < 0) return MOE_EUNSUPPORTED;
    const long n_pairs = (long)T * k;
    const int slots = (int)(n_pairs < E ? n_pairs : E);
    dim3 g1((unsigned)slots * (I / 16)), g2((unsigned)slots * ((H + 63) / 64));
    int rc = fmt == MOE_W_MXFP4
                 ? launch_gate_up<MOE_W_MXFP4>(spw, g1, s, x, sorted_pair, offsets, experts, k, H,
                                               I, E, act)
                 : launch_gate_up<MOE_W_BF16>(spw, g1, s, x, sorted_pair, offsets, experts, k, H, I,
                                              E, act);
    if (rc) return rc;
    if (fmt == MOE_W_MXFP4)
        return y_is_fp32 ? launch_down<MOE_W_MXFP4, true>(spk, g2, s, act, sorted_pair, offsets,
                                                          experts, H, I, E, y)
                         : launch_down<MOE_W_MXFP4, false>(spk, g2, s, act, sorted_pair, offsets,
                                                           experts, H, I, E, y);
    return y_is_fp32 ? launch_down<MOE_W_BF16, true>(spk, g2, s, act, sorted_pair, offsets, experts,
                                                     H, I, E, y)
                     : launch_down<MOE_W_BF16, false>(spk, g2, s, act, sorted_pair, offsets,
                                                      experts, H, I, E, y);
}

}  // namespace moe
