// Prefill-shaped grouped SwiGLU expert FFN: hundreds of tokens per expert,
// so the contraction is dense enough for the matrix cores to bound it.
//
// In prefill almost every expert receives tokens (winzheng.com page, "Why Now
// of All Times": large prefill batches route to nearly all experts in every
// layer). Each expert's block is a grouped matrix product; this kernel tiles
// it for bf16 32x32x16 MFMA, decoding the MXFP4 weights in registers.
//
// Tile (one 512-thread workgroup: 8 wavefronts, two per SIMD, each 64 weight
// rows x 64 token rows): 256 weight rows x 128 token rows of one expert over
// the full contraction K, in 128-column slabs
// that stream straight from global memory into a 3-stage LDS ring (two slabs
// in flight while one is multiplied; one barrier per slab):
//   - weights (MFMA operand A, kernel MXFP4 layout): the tile's 16 row blocks
//     (16 rows x 128 columns = one 1 KB block each) are copied as they are;
//     each wavefront decodes its 4 blocks in registers right before use;
//   - tokens (operand B): the tile's 128 rows (gathered x rows in stage 1,
//     activation rows in stage 2) with the 16-byte column chunks XOR-swizzled
//     by row so the fragment reads hit distinct banks.
// (On gfx950 the 32x32x16 bf16 MFMA issues at twice the 16x16x32 rate.)
// Stage 1 tile rows: 128 gate rows and the matching 128 up rows (32 + 32 per
// wavefront), so SwiGLU happens in registers. Stage 2 tile rows: 256 W2 rows.
// Tiles are numbered per expert (token tile major, weight tile minor) and the
// numbering is split into 8 contiguous ranges, one per XCD (workgroup b runs
// on XCD b % 8), so an expert's tiles share one XCD's L2.
#include <math.h>

#include "common.hpp"

namespace moe {

constexpr int kPreTok = 128;      // token rows per tile
constexpr int kPreThreads = 512;
constexpr int kSlabBytes = 256;   // one token row's slab: 128 bf16

__device__ __forceinline__ float silu_mul_p(float g, float u) {
    return g / (1.0f + __expf(-g)) * u;
}

struct PreArgs {
    const uint16_t *src;          // token operand rows: x [T][H] or act [T*k][I]
    const int32_t *sorted_pair;
    const int32_t *offsets;
    const moe_expert_w *experts;
    void *out;                    // act (stage 1) or y (stage 2)
    int k, K, H, I, E;
    int ntiles_w;                 // weight tiles per expert
};

// Expert, token-tile and weight-tile of tile q (all lanes get the same) and
// the total number of tiles. Returns false if q is past the last tile.
__device__ __forceinline__ bool pre_find_tile(const PreArgs &A, long q, int &e, int &mt, int &nt,
                                              long &total) {
    const int lane = lane_id();
    long base = 0;
    e = -1;
    for (int e0 = 0; e0 < A.E; e0 += kWave) {
        const int ee = e0 + lane;
        long mtiles = 0;
        if (ee < A.E) mtiles = (A.offsets[ee + 1] - A.offsets[ee] + kPreTok - 1) / kPreTok;
        const long tiles = mtiles * A.ntiles_w;
        // inclusive prefix over the wavefront
        long incl = tiles;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const long o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        const long excl = base + incl - tiles;
        const bool hit = e < 0 && tiles > 0 && q >= excl && q < excl + tiles;
        const uint64_t hm = __ballot(hit);
        if (hm) {
            const int src = __ffsll((long long)hm) - 1;
            e = e0 + src;
            const long local = q - __shfl(excl, src);
            mt = (int)(local / A.ntiles_w);
            nt = (int)(local - (long)mt * A.ntiles_w);
        }
        base += __shfl(incl, kWave - 1);
    }
    total = base;
    return e >= 0;
}

// LDS of one slab stage: the tile's 128 token rows (swizzled 16-byte chunks)
// and its 16 weight blocks (1 KB codes + 64 B scales each).
struct PreStage {
    uint8_t tok[kPreTok * kSlabBytes];
    uint8_t wcode[16][1024];
    uint8_t wscale[16][64];
};
constexpr int kPreStages = 3;                  // computing s, landing s+1 and s+2

#define MOE_LDS __attribute__((address_space(3)))

// Direct global -> LDS copies: lane l's 16 bytes land at dst + 16 l (dst is
// wavefront-uniform).
__device__ __forceinline__ void lds_dma16(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds((const MOE_GLOBAL void *)src, (MOE_LDS void *)dst, 16, 0, 0);
}

// Waits until at most n of this wavefront's vector-memory operations are
// outstanding (n < 64). gfx9 s_waitcnt fields: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt_hi[15:14].
template <int N>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// This wavefront's copies of slab s into stage st (8 wavefronts):
//  tokens: copy u (u < 4) covers tile rows 16w + 4u .. +3 (lane l: row + l/16,
//          LDS slot l%16, which holds global 16-byte chunk slot ^ (row & 15));
//  codes : tile-local blocks 2w, 2w+1 (1 KB each, copied as they are);
//  scales: wavefront 7 copies all 16 blocks' 64-byte scale rows (lane l:
//          bytes 16(l%4) .. +15 of block l/4).
// Returns the number of copies issued (6, or 7 on wavefront 7).
__device__ __forceinline__ void pre_issue(PreStage &st, int s, int w, int lane,
                                          const uint16_t *const (&trow)[4], const uint8_t *wcodes,
                                          const uint8_t *wscales, const long (&rbw)[2],
                                          long rbs, int nslab) {
    const int r_lane = lane >> 4, slot = lane & 15;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int r = 16 * w + 4 * u + r_lane;
        const int c16 = slot ^ (r & 15);
        lds_dma16(trow[u] + s * 128 + c16 * 8, &st.tok[(16 * w + 4 * u) * kSlabBytes]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
        lds_dma16(wcodes + ((size_t)rbw[u] * nslab + s) * 1024 + lane * 16,
                  &st.wcode[2 * w + u][0]);
    if (w == 7)
        lds_dma16(wscales + ((size_t)rbs * nslab + s) * 64 + (lane & 3) * 16, &st.wscale[0][0]);
}

// Fragments of half a slab (4 MFMA steps of 16 columns) for this
// wavefront's 64 weight rows (two 32-row groups = tile-local blocks 4wn ..
// 4wn+3) and 64 tokens (two 32-token groups). Step k reads columns 16k ..
// 16k+15; lane l supplies 8 of them (8(l/32) ..): for the weights, row l%32 of
// the group sits in block l/16 as lane-chunk (l%16) + 16(k/2), bytes
// 8(k%2) + 4(l/32) .. +3; for the tokens, row l%32 of the token group, 16-byte
// chunk 2k + l/32 (swizzled).
struct PreFrag {
    u32x4 tb[4][2];
    uint32_t wq[4][2];
    uint32_t sb[2];         // scale bytes of the half's two 32-column blocks, per weight group
};

__device__ __forceinline__ void pre_read(const PreStage &st, PreFrag &f, int half, int wm, int wn,
                                         int lane) {
    const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int k = 4 * half + kk;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int r = wm * 64 + t * 32 + r32;
            const int slot = (2 * k + h) ^ (r & 15);
            f.tb[kk][t] = *reinterpret_cast<const u32x4 *>(&st.tok[r * kSlabBytes + slot * 16]);
        }
#pragma unroll
        for (int gq = 0; gq < 2; ++gq) {
            const int wb = 4 * wn + 2 * gq + (r32 >> 4);
            f.wq[kk][gq] = *reinterpret_cast<const uint32_t *>(
                &st.wcode[wb][((r32 & 15) + 16 * (k >> 1)) * 16 + 8 * (k & 1) + 4 * h]);
        }
    }
#pragma unroll
    for (int gq = 0; gq < 2; ++gq) {
        const int wb = 4 * wn + 2 * gq + (r32 >> 4);
        // this half's 32-column blocks are 2 half and 2 half + 1
        f.sb[gq] = (uint32_t)st.wscale[wb][(r32 & 15) + 32 * half] |
                   ((uint32_t)st.wscale[wb][(r32 & 15) + 32 * half + 16] << 8);
    }
}

__device__ __forceinline__ void pre_math(const PreFrag &f, f32x16 (&acc)[2][2]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int gq = 0; gq < 2; ++gq) {
            const float sc = e8m0_to_f32((f.sb[gq] >> (8 * (kk >> 1))) & 0xFFu);
            const bf16x8 aw = dequant8_fp4(f.wq[kk][gq], sc);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                acc[gq][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw, as_bf16x8(f.tb[kk][t]),
                                                                    acc[gq][t], 0, 0, 0);
        }
    }
}

// 16-row weight block (within the stage's matrix) of tile-local block wb of
// weight tile nt (wb = 4q + b, q = the wavefront's weight quarter): stage 1 ->
// q's two gate blocks for b < 2 and the matching up blocks for b >= 2 (act
// columns nt*128 + 32q .. +31); stage 2 -> 16 consecutive W2 blocks.
template <int STAGE>
__device__ __forceinline__ long pre_block(const PreArgs &A, int nt, int wb) {
    const int qq = wb >> 2, b = wb & 3;
    if (STAGE == 1)
        return b < 2 ? (long)nt * 8 + qq * 2 + b : (long)A.I / 16 + nt * 8 + qq * 2 + (b - 2);
    return (long)nt * 16 + wb;
}

template <int STAGE, bool YF32>
__global__ __launch_bounds__(kPreThreads) void ffn_pre_kernel(PreArgs A) {
    __shared__ __attribute__((aligned(16))) PreStage lds[kPreStages];
    const int tid = threadIdx.x, lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wv >> 2, wn = wv & 3;     // token half, weight quarter

    // total tiles, then this workgroup's tile (XCD-aware numbering)
    int e, mt, nt;
    long total;
    pre_find_tile(A, 0, e, mt, nt, total);
    const long per = (total + 7) / 8;
    const long q = (long)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if ((long)(blockIdx.x >> 3) >= per || q >= total) return;
    pre_find_tile(A, q, e, mt, nt, total);

    const int row0 = A.offsets[e];
    const int n_e = A.offsets[e + 1] - row0;
    const int tok0 = mt * kPreTok;
    const moe_expert_w W = A.experts[e];
    const uint8_t *wcodes = reinterpret_cast<const uint8_t *>(STAGE == 1 ? W.w13 : W.w2);
    const uint8_t *wscales = STAGE == 1 ? W.s13 : W.s2;
    const int nslab = A.K / 128;

    // blocks whose codes this wavefront copies (tile-local 2wv, 2wv+1) and the
    // block whose scales this lane copies on wavefront 7 (tile-local lane/4)
    long rbw[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) rbw[u] = pre_block<STAGE>(A, nt, 2 * wv + u);
    const long rbs = pre_block<STAGE>(A, nt, lane >> 2);
    // token rows this lane copies: 16 wv + 4u + lane/16 (u < 4)
    const uint16_t *trow[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        int r = tok0 + 16 * wv + 4 * u + (lane >> 4);
        r = r < n_e ? r : n_e - 1;              // rows past the expert's end repeat its last row
        if (STAGE == 1) trow[u] = A.src + (size_t)(A.sorted_pair[row0 + r] / A.k) * A.K;
        else trow[u] = A.src + (size_t)(row0 + r) * A.K;
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int gq = 0; gq < 2; ++gq)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[gq][t][i] = 0.0f;

    // Software pipeline over half slabs: fragments of the next half are read
    // from LDS while the current half is multiplied from registers. One
    // barrier per slab, between its two halves: before it every wavefront has
    // slab s in registers and has seen slab s + 1 land; after it slab s + 1 is
    // visible to all and slab s's stage takes the copy of slab s + 3. (A bare
    // barrier: a fenced __syncthreads would also wait for the copies still in
    // flight.)
    const int nw = wv == 7 ? 7 : 6;          // copies per slab issued by this wavefront
    auto wait_copies = [&](int later) {       // wait until only `later` slabs' copies remain
        const int n = later * nw;
        if (n == 0) wait_vm<0>();
        else if (n == 6) wait_vm<6>();
        else if (n == 7) wait_vm<7>();
        else if (n == 12) wait_vm<12>();
        else wait_vm<14>();
    };
    for (int i = 0; i < kPreStages && i < nslab; ++i)
        pre_issue(lds[i], i, wv, lane, trow, wcodes, wscales, rbw, rbs, nslab);
    wait_copies(nslab - 1 < kPreStages - 1 ? nslab - 1 : kPreStages - 1);
    __builtin_amdgcn_s_barrier();
    PreFrag fa, fb;
    pre_read(lds[0], fa, 0, wm, wn, lane);
    for (int s = 0; s < nslab; ++s) {
        pre_read(lds[s % kPreStages], fb, 1, wm, wn, lane);
        pre_math(fa, acc);
        if (s + 1 < nslab) {
            __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): slab s fully in registers
            wait_copies(s + 2 < nslab ? 1 : 0);      // slab s + 1 landed
            __builtin_amdgcn_s_barrier();
            if (s + 3 < nslab)
                pre_issue(lds[s % kPreStages], s + 3, wv, lane, trow, wcodes, wscales, rbw, rbs,
                          nslab);
            pre_read(lds[(s + 1) % kPreStages], fa, 0, wm, wn, lane);
        }
        pre_math(fb, acc);
    }

    // epilogue: for token group t the lane holds token 64wm + 32t + lane%32 and,
    // in weight group gq, rows 8(i/4) + 4(lane/32) + i%4 (i < 16) of the group
    const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int r = tok0 + wm * 64 + t * 32 + r32;
        if (r >= n_e) continue;
        if (STAGE == 1) {
            // group 0 = 32 gate rows, group 1 = the matching 32 up rows
            uint16_t *act = reinterpret_cast<uint16_t *>(A.out) + (size_t)(row0 + r) * A.I +
                            nt * 128 + wn * 32 + 4 * h;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int i0 = 4 * q4;
                uint2 pk;
                pk.x = pack_bf16x2(silu_mul_p(acc[0][t][i0], acc[1][t][i0]),
                                   silu_mul_p(acc[0][t][i0 + 1], acc[1][t][i0 + 1]));
                pk.y = pack_bf16x2(silu_mul_p(acc[0][t][i0 + 2], acc[1][t][i0 + 2]),
                                   silu_mul_p(acc[0][t][i0 + 3], acc[1][t][i0 + 3]));
                *reinterpret_cast<uint2 *>(act + 8 * q4) = pk;
            }
        } else {
            const size_t prow = (size_t)A.sorted_pair[row0 + r] * A.H + nt * 256 + wn * 64 + 4 * h;
#pragma unroll
            for (int gq = 0; gq < 2; ++gq)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int i0 = 4 * q4;
                    const size_t off = prow + gq * 32 + 8 * q4;
                    if (YF32) {
                        f32x4 v = {acc[gq][t][i0], acc[gq][t][i0 + 1], acc[gq][t][i0 + 2],
                                   acc[gq][t][i0 + 3]};
                        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(A.out) + off) = v;
                    } else {
                        uint2 pk;
                        pk.x = pack_bf16x2(acc[gq][t][i0], acc[gq][t][i0 + 1]);
                        pk.y = pack_bf16x2(acc[gq][t][i0 + 2], acc[gq][t][i0 + 3]);
                        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(A.out) + off) = pk;
                    }
                }
        }
    }
}

// Tiled path needs whole 128-row weight tiles in stage 1 (I % 128) and
// 256-row tiles in stage 2 (H % 256), and whole 128-column slabs.
bool ffn_prefill_supported(int fmt, int H, int I) {
    return fmt == MOE_W_MXFP4 && I % 128 == 0 && H % 256 == 0;
}

template <int STAGE, bool YF32>
static int launch_pre(hipStream_t s, PreArgs A, long n_pairs) {
    // upper bound on tiles: sum_e ceil(count_e / 128) <= n_pairs / 128 + E
    const long mt_max = n_pairs / kPreTok + A.E;
    const long tiles_max = mt_max * A.ntiles_w;
    const long grid = ((tiles_max + 7) / 8) * 8;
    if (grid > 0x7FFFFFFFL) return MOE_EUNSUPPORTED;
    MOE_TIMED(s, STAGE == 1 ? K_PRE_GATE_UP : K_PRE_DOWN,
              hipLaunchKernelGGL((ffn_pre_kernel<STAGE, YF32>), dim3((unsigned)grid),
                                 dim3(kPreThreads), 0, s, A));
    return check_launch();
}

int ffn_prefill(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
                const moe_expert_w *experts, int fmt, int T, int k, int H, int I, int E, void *y,
                int y_is_fp32, uint16_t *act, hipStream_t s) {
    if (!ffn_prefill_supported(fmt, H, I)) return MOE_EUNSUPPORTED;
    const long n = (long)T * k;
    PreArgs a1{x, sorted_pair, offsets, experts, act, k, H, H, I, E, I / 128};
    int rc = launch_pre<1, false>(s, a1, n);
    if (rc) return rc;
    PreArgs a2{act, sorted_pair, offsets, experts, y, k, I, H, I, E, H / 256};
    return y_is_fp32 ? launch_pre<2, true>(s, a2, n) : launch_pre<2, false>(s, a2, n);
}

}  // namespace moe
