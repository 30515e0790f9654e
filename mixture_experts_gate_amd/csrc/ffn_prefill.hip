// Prefill-shaped grouped SwiGLU expert FFN: hundreds of tokens per expert,
// so the contraction is dense enough for the matrix cores to bound it.
//
// In prefill almost every expert receives tokens (winzheng.com page, "Why Now
// of All Times": large prefill batches route to nearly all experts in every
// layer). Each expert's block is a grouped matrix product, tiled here for the
// block-scaled MFMA of gfx950 (v_mfma_scale_f32_16x16x128_f8f6f4), which
// multiplies the MXFP4 weights as they are stored: E2M1 codes with one E8M0
// scale per 32 elements, no decode in registers.
//
// The token operand is carried as two FP8 (E4M3) terms with one E8M0 scale
// per 32 elements: hi = fp8(x / 2^e), lo = fp8(32 (x / 2^e - hi)) with scale
// 2^(e-5), e = floor(log2 max|x|) - 7 over the 32-element block. hi holds x to
// 2^-4 relative, lo the remainder to another 2^-4, so hi + lo is within
// 2^-8 |x| + 2^-22 max|block| of x (bf16 keeps 2^-9; the second term covers
// elements so small that a term falls in E4M3's subnormal range); both terms
// run through the FP8 x FP4 matrix pipe, whose rate is twice bf16's, so the
// pair costs what one bf16 product would, and the weights need no conversion. x is split once per token
// by a row pass; the activation a = silu(g) * u is split by the gate/up
// kernel's epilogue as it is produced.
//
// Tile (one 256-thread workgroup: 4 wavefronts, one per SIMD, each 32 tokens x
// 128 weight rows; two workgroups share a compute unit): 64 tokens x 256
// weight rows of one expert over the full contraction K, in 128-column slabs
// copied straight from global memory into a 2-stage LDS ring (one slab in
// flight while one is multiplied; one barrier per slab). 64-token tiles halve
// the padding of each expert's last tile. Every operand lands in LDS in the order the matrix core reads it,
// so each fragment read is one contiguous 16-byte-per-lane LDS read:
//   - weights (operand A, kernel MXFP4 layout): 16 row blocks of 16 rows x 128
//     columns (1 KB codes + 64 B scales each), copied as they are;
//   - tokens (operand B): per 16-token block, term and 64-column half, lane l
//     holds token l%16, columns 64 half + 16(l/16) .. +15;
//   - token scales: lane l of a token block holds token l%16's four scales.
// Stage 1 rows: 128 gate rows and the matching 128 up rows (64 + 64 per
// wavefront), so SwiGLU happens in registers. Stage 2 rows: 256 W2 rows.
// Tiles are numbered per expert (token tile major, weight tile minor) and the
// numbering is split into 8 contiguous ranges, one per XCD (workgroup b runs
// on XCD b % 8), so an expert's tiles share one XCD's L2.
#include <math.h>

#include <type_traits>

#include "common.hpp"

namespace moe {

constexpr int kPreTok = 64;       // tokens per tile
constexpr int kPreThreads = 256;  // four wavefronts; two workgroups share a compute unit
constexpr int kLoShift = 5;       // lo term scale = hi scale / 2^5

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

// silu(g) * u with the hardware reciprocal (about 1 ulp)
__device__ __forceinline__ float silu_mul_p(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// ---------------------------------------------------------- two-term FP8 --

// Block exponent e (as the hi scale's E8M0 byte, e + 127) for a block whose
// largest magnitude is amax: e = floor(log2 amax) - 7 puts the block maximum
// in [128, 256), inside E4M3's range (448). Clamped to [5, 254] so the lo
// scale byte (hi - 5) stays a valid E8M0 value; blocks below 2^-115 lose
// relative precision, which no bf16 activation of interest reaches.
__device__ __forceinline__ int split_scale_byte(float amax) {
    const int eb = (int)((__float_as_uint(amax) >> 23) & 0xFFu);   // biased exponent
    int b = eb - 7;                                                 // (eb - 127 - 7) + 127
    b = b < kLoShift ? kLoShift : b;
    return b > 254 ? 254 : b;
}

// 1 / 2^e for hi scale byte b (2^(127 - b), exact).
__device__ __forceinline__ float split_inv_scale(int b) {
    return __uint_as_float((uint32_t)(254 - b) << 23);
}

// Two values (already divided by the hi scale) -> two hi and two lo E4M3
// bytes, packed in the low 16 bits of hi / lo.
__device__ __forceinline__ void split_pair(float v0, float v1, uint32_t &hi, uint32_t &lo) {
    const int h = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
    const float r0 = v0 - __builtin_amdgcn_cvt_f32_fp8(h, 0);     // exact (Sterbenz)
    const float r1 = v1 - __builtin_amdgcn_cvt_f32_fp8(h, 1);
    const int l = __builtin_amdgcn_cvt_pk_fp8_f32(r0 * 32.0f, r1 * 32.0f, 0, false);
    hi = (uint32_t)h & 0xFFFFu;
    lo = (uint32_t)l & 0xFFFFu;
}

// Four values -> four hi and four lo bytes.
__device__ __forceinline__ void split_quad(const float (&v)[4], float inv, uint32_t &hi,
                                           uint32_t &lo) {
    uint32_t h0, l0, h1, l1;
    split_pair(v[0] * inv, v[1] * inv, h0, l0);
    split_pair(v[2] * inv, v[3] * inv, h1, l1);
    hi = h0 | (h1 << 16);
    lo = l0 | (l1 << 16);
}

// Row split of bf16 rows [rows][K] into hi [rows][K], lo [rows][K] and hi
// scale bytes [rows][K/32]. Four threads per 32-element block.
// Token-tile map of the tiled kernels: map[0] = M, the number of 64-token
// tiles over all experts; map[1 + m] = e | (mt << 16) for the m-th tile in
// expert order (tile mt of expert e). The always-on shared expert, when the
// launch carries it, is expert E with sh_rows rows (the tokens in order).
// One 256-thread workgroup.
__device__ void build_tile_map(const int32_t *__restrict__ offsets, int E, int sh_rows,
                               int32_t *__restrict__ map) {
    __shared__ int wsum[4];
    const int t = threadIdx.x, lane = lane_id(), w = t / kWave;
    int run = 0;   // tiles of the experts before this chunk
    for (int e0 = 0; e0 <= E; e0 += 256) {
        const int e = e0 + t;
        const int rows = e < E ? offsets[e + 1] - offsets[e] : e == E ? sh_rows : 0;
        const int tiles = (rows + kPreTok - 1) / kPreTok;
        int incl = tiles;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        if (lane == kWave - 1) wsum[w] = incl;
        __syncthreads();
        int wbase = 0, total = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wbase += i < w ? wsum[i] : 0;
            total += wsum[i];
        }
        const int base = run + wbase + incl - tiles;
        for (int mt = 0; mt < tiles; ++mt) map[1 + base + mt] = e | (mt << 16);
        run += total;
        __syncthreads();
    }
    if (t == 0) map[0] = run;
}

// The last workgroup (one past the row blocks) builds the token-tile map.
__global__ __launch_bounds__(256) void split_rows_kernel(const uint16_t *__restrict__ src,
                                                         long nblk, uint8_t *__restrict__ hi,
                                                         uint8_t *__restrict__ lo,
                                                         uint8_t *__restrict__ sc,
                                                         const int32_t *__restrict__ offsets,
                                                         int E, int sh_rows,
                                                         int32_t *__restrict__ map) {
    if (blockIdx.x == gridDim.x - 1) {
        build_tile_map(offsets, E, sh_rows, map);
        return;
    }
    // four threads per 32-element block, eight elements each, so that loads
    // and stores are contiguous across the wavefront; the block maximum meets
    // over the four lanes of a DPP quad (a block's threads are one quad)
    const long g = (long)blockIdx.x * 256 + threadIdx.x;
    const long b = g >> 2;
    const int qd = (int)(g & 3);
    const bool ok = b < nblk;
    const u32x4 v = ok ? load_nt16(src + b * 32 + 8 * qd) : u32x4{0, 0, 0, 0};
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
        amax = fmaxf(amax, fmaxf(fabsf(bf16_bits_to_f32(v[c] & 0xFFFFu)),
                                 fabsf(bf16_bits_to_f32(v[c] >> 16))));
    // quad_perm [1,0,3,2], then [2,3,0,1]
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0xB1,
                                                                  0xF, 0xF, false)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x4E,
                                                                  0xF, 0xF, false)));
    const int sb = split_scale_byte(amax);
    const float inv = split_inv_scale(sb);
    const float v0[4] = {bf16_bits_to_f32(v[0] & 0xFFFFu), bf16_bits_to_f32(v[0] >> 16),
                         bf16_bits_to_f32(v[1] & 0xFFFFu), bf16_bits_to_f32(v[1] >> 16)};
    const float v1[4] = {bf16_bits_to_f32(v[2] & 0xFFFFu), bf16_bits_to_f32(v[2] >> 16),
                         bf16_bits_to_f32(v[3] & 0xFFFFu), bf16_bits_to_f32(v[3] >> 16)};
    uint2 oh, ol;
    split_quad(v0, inv, oh.x, ol.x);
    split_quad(v1, inv, oh.y, ol.y);
    if (!ok) return;
    *reinterpret_cast<uint2 *>(hi + b * 32 + 8 * qd) = oh;
    *reinterpret_cast<uint2 *>(lo + b * 32 + 8 * qd) = ol;
    if (qd == 0) sc[b] = (uint8_t)sb;
}

// ------------------------------------------------------------ GEMM tiles --

struct PreArgs {
    const uint8_t *bhi, *blo, *bsc;   // token operand: hi/lo rows [.][K], scales [.][K/32]
    const int32_t *sorted_pair;
    const int32_t *offsets;
    const moe_expert_w *experts;
    void *out;                        // stage 2: y
    uint8_t *ohi, *olo, *osc;         // stage 1: activation hi/lo rows [n][I], scales [n][I/32]
    const int32_t *tile_map;          // token-tile map (build_tile_map)
    const moe_expert_w *shared;       // the shared expert (expert index E), or NULL
    int k, K, H, I, E, T;
    int ntiles_w;                     // weight tiles per expert
    int nt_group;                     // consecutive weight tiles per workgroup (divides ntiles_w)
};

// LDS of one slab stage (34048 bytes; two stages per workgroup, so two
// workgroups fit a compute unit's 160 KB).
//   tok   : [term hi/lo][16-token block] 16 rows x 128 bytes; the 16-byte chunk c
//           of row r sits at position c ^ ((r / 2) % 8), so the 16 lanes that
//           read one chunk of 16 rows hit 16 different 16-byte bank groups;
//   tsc   : the 64 tokens' 4 scale bytes of this slab;
//   wcode / wscale: the tile's 16 weight blocks, kernel layout.
// FP8 weights (one byte per element) take 2 KB per weight block: the stage
// is then 50 KB and one workgroup fits a compute unit.
constexpr int wblock_bytes(int fmt) { return fmt == MOE_W_FP8 ? 2048 : 1024; }

template <int FMT>
struct PreStage {
    uint8_t tok[2][4][2048];
    uint8_t wcode[16][wblock_bytes(FMT)];
    uint8_t tsc[kPreTok][4];
    uint8_t wscale[16][64];
};
constexpr int kPreStages = 2;     // computing s, landing s+1

__device__ __forceinline__ int tok_swz(int r) { return (r >> 1) & 7; }

// Per-lane copy sources of one tile (slab 0; slab s adds s * 128 bytes to a
// token row, s * 4 to a scale row, s * 1024 / s * 64 to a weight block).
struct PreSrc {
    const uint8_t *thi[2], *tlo[2];   // token block w, rows 8u + lane/8: the lane's 16-byte chunk
    const uint8_t *tsc;               // wavefront 0: scale row of token lane
    const uint8_t *wc[4];             // blocks 4w .. 4w+3: codes + 16 lane
    const uint8_t *ws;                // wavefront 1: scales of block lane/4 + 16 (lane%4)
};

// This wavefront's copies of slab s into stage st (4 wavefronts): its token
// block's two terms (8 rows x 128 bytes per copy), weight blocks 4w .. 4w+3,
// on wavefront 0 the token scales, on wavefront 1 the 16 weight blocks' scale rows.
// woff: byte offset of this weight tile's codes from the group's first tile's
// (its scales sit at woff / 16).
template <int FMT>
__device__ __forceinline__ void pre_issue(PreStage<FMT> &st, int s, int w, const PreSrc &p,
                                          size_t woff) {
    constexpr int WB = wblock_bytes(FMT);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        lds_dma16(p.thi[u] + s * 128, &st.tok[0][w][u * 1024]);
        lds_dma16(p.tlo[u] + s * 128, &st.tok[1][w][u * 1024]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        lds_dma16(p.wc[u] + woff + (size_t)s * WB, &st.wcode[4 * w + u][0]);
        if (WB == 2048) lds_dma16(p.wc[u] + woff + (size_t)s * WB + 1024, &st.wcode[4 * w + u][1024]);
    }
    if (w == 0) lds_dma4(p.tsc + s * 4, &st.tsc[0][0]);
    if (FMT == MOE_W_MXFP4 && w == 1)
        lds_dma16(p.ws + woff / 16 + (size_t)s * 64, &st.wscale[0][0]);
}

// One slab's operands for one wavefront: its 8 weight blocks and its two
// 16-token blocks (both terms, both halves), with the lane's scale bytes.
template <int FMT>
struct PreFrag {
    u32x4 w[8];
    u32x4 w2[FMT == MOE_W_FP8 ? 8 : 1];   // FP8: the lane's second 16 bytes of each block
    uint32_t ws[8];
    i32x8 t[2][2];                // [token block][term]; elements 0-3 / 4-7 = column half 0 / 1
    uint32_t ts[2];
};

// LDS block (of the stage's 16) holding this wavefront's weight block b:
// stage 1 -> gate blocks 4wn .. 4wn+3 then the matching up blocks 8 + 4wn ..;
// stage 2 -> blocks 8wn .. 8wn+7.
template <int STAGE>
__device__ __forceinline__ int lds_block(int wn, int b) {
    if (STAGE == 1) return b < 4 ? 4 * wn + b : 8 + 4 * wn + (b - 4);
    return 8 * wn + b;
}

// Token fragment positions of this lane (row lane%16 of a block, chunks
// lane/16 and lane/16 + 4 of the row: columns 16(lane/16) and 64 + 16(lane/16)).
struct TokPos {
    int a0, a1;
    __device__ __forceinline__ explicit TokPos(int lane) {
        const int r = lane & 15, c0 = lane >> 4;
        a0 = 128 * r + 16 * (c0 ^ tok_swz(r));
        a1 = 128 * r + 16 * ((c0 + 4) ^ tok_swz(r));
    }
};

template <int STAGE, int FMT>
__device__ __forceinline__ void pre_read(const PreStage<FMT> &st, PreFrag<FMT> &f, int wm, int wn,
                                         int lane, const TokPos &tp) {
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const int lb = lds_block<STAGE>(wn, b);
        if constexpr (FMT == MOE_W_FP8) {
            // an 8-bit operand lane holds columns 16g..16g+15 (bytes 0-15) and
            // 64+16g.. (bytes 16-31), g = lane / 16, like the token operand;
            // the block stores each row's columns 32h..32h+31 as one 32-byte
            // piece at (16h + row) * 32
            const int r = lane & 15, g = lane >> 4;
            const int a0 = ((g >> 1) * 16 + r) * 32 + 16 * (g & 1);
            const int a1 = ((2 + (g >> 1)) * 16 + r) * 32 + 16 * (g & 1);
            f.w[b] = *reinterpret_cast<const u32x4 *>(&st.wcode[lb][a0]);
            f.w2[b] = *reinterpret_cast<const u32x4 *>(&st.wcode[lb][a1]);
        } else {
            f.w[b] = *reinterpret_cast<const u32x4 *>(&st.wcode[lb][16 * lane]);
            f.ws[b] = st.wscale[lb][lane];
        }
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int term = 0; term < 2; ++term) {
            const uint8_t *blk = st.tok[term][2 * wm + tb];
            f.t[tb][term].lo = *reinterpret_cast<const i32x4 *>(blk + tp.a0);
            f.t[tb][term].hi = *reinterpret_cast<const i32x4 *>(blk + tp.a1);
        }
        f.ts[tb] = st.tsc[16 * (2 * wm + tb) + (lane & 15)][lane >> 4];
    }
}

// nvb: this wavefront's token blocks that hold rows of the expert (2, 1 or
// 0; wavefront-uniform): a block wholly past the expert's last row (in the
// expert's last, partial tile) issues no matrix instructions.
template <int FMT, int NTB>
__device__ __forceinline__ void pre_math_tb(const PreFrag<FMT> &f, f32x4 (&acc)[8][2]) {
#pragma unroll
    for (int term = 0; term < 2; ++term)
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const i32x4 w4 = __builtin_bit_cast(i32x4, f.w[b]);
            i32x8 a;
            if constexpr (FMT == MOE_W_FP8) {
                const i32x4 w4b = __builtin_bit_cast(i32x4, f.w2[b]);
                a = __builtin_shufflevector(w4, w4b, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
                // E2M1 operand: only the low four dwords are read
                a = __builtin_shufflevector(w4, w4, 0, 1, 2, 3, -1, -1, -1, -1);
            }
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                const int tsc = (int)f.ts[tb] - (term ? kLoShift : 0);
                // A: E2M1 (format 4) with its E8M0 block scale, or E4M3 (format
                // 0) with unit scale 127; B: E4M3 (format 0)
                if constexpr (FMT == MOE_W_FP8)
                    acc[b][tb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        a, f.t[tb][term], acc[b][tb], 0, 0, 0, 127, 0, tsc);
                else
                    acc[b][tb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        a, f.t[tb][term], acc[b][tb], 4, 0, 0, (int)f.ws[b], 0, tsc);
            }
        }
}

// 16-row weight block (within the stage's matrix) copied into LDS block lb of
// weight tile nt: stage 1 -> gate blocks nt*8 + lb (lb < 8), up blocks I/16 +
// nt*8 + lb - 8; stage 2 -> W2 blocks nt*16 + lb.
template <int STAGE>
__device__ __forceinline__ long pre_block(const PreArgs &A, int nt, int lb) {
    if (STAGE == 1) return lb < 8 ? (long)nt * 8 + lb : (long)A.I / 16 + nt * 8 + (lb - 8);
    return (long)nt * 16 + lb;
}

// Barrier without a memory fence (a fenced __syncthreads would also wait for
// the copies still in flight); the empty asm statements keep the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Double-buffered slab loop over one weight tile; the ring runs on across the
// workgroup's tiles, slab g (counted over the group) sitting in stage g % 2.
// At the top of a slab this wavefront's copies of it have landed (they are
// the only loads in flight), and after the barrier every wavefront's have, and
// every wavefront has finished reading the previous slab, whose stage then
// receives the next one (the next tile's first slab after a tile's last). The
// two workgroups on a compute unit interleave: one's copies, fragment reads,
// barrier waits and epilogue overlap the other's matrix instructions.
// `first` runs once, after the first slab's barrier and copies: the previous
// tile's deferred output stores go there, so that the wait at the top of the
// first slab does not also wait for them to complete.
// NVB: this wavefront's token blocks that hold rows of the expert (2, 1 or
// 0): a block wholly past the expert's last row (in the expert's last,
// partial tile) issues no matrix instructions. A template argument, chosen
// once per workgroup, so that the slab loop has no branch around them.
template <int STAGE, int FMT, int NVB, class First>
__device__ __forceinline__ void pre_mainloop(PreStage<FMT> (&lds)[kPreStages], f32x4 (&acc)[8][2],
                                             int n, int g0, int wv, int wm, int wn, int lane,
                                             const PreSrc &src, size_t woff, size_t woff_next,
                                             bool has_next, First &&first) {
    PreFrag<FMT> F;
    const TokPos tp(lane);
    for (int j = 0; j < n; ++j) {
        const int st = (g0 + j) & 1;
        wait_vm<0>();
        bare_barrier();
        if (j + 1 < n) pre_issue<FMT>(lds[st ^ 1], j + 1, wv, src, woff);
        else if (has_next) pre_issue<FMT>(lds[st ^ 1], 0, wv, src, woff_next);
        if (j == 0) first();
        pre_read<STAGE, FMT>(lds[st], F, wm, wn, lane, tp);
        pre_math_tb<FMT, NVB>(F, acc);
    }
}

// Epilogue of weight tile nt: for token block tb the lane holds token
// 32wm + 16tb + lane%16 and, in weight block b, rows 4(lane/16) + i (i < 4) of
// the block.
// Stage 2, bf16 y: a tile's outputs packed, and stored later (pre_store_y).
struct PreOut {
    uint2 pk[2][8];
    int nt;
};

__device__ __forceinline__ void pre_pack_y(const f32x4 (&acc)[8][2], int nt, PreOut &o) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            o.pk[tb][b].x = pack_bf16x2(acc[b][tb][0], acc[b][tb][1]);
            o.pk[tb][b].y = pack_bf16x2(acc[b][tb][2], acc[b][tb][3]);
        }
    o.nt = nt;
}

__device__ __forceinline__ void pre_store_y(const PreArgs &A, const PreOut &o, int tok0, int n_e,
                                            int wm, int wn, int lane, const int (&prow_tb)[2]) {
    const int g4 = lane >> 4;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int r = tok0 + 32 * wm + 16 * tb + (lane & 15);
        if (r >= n_e) continue;
        const size_t prow = (size_t)prow_tb[tb] * A.H + o.nt * 256 + 128 * wn + 4 * g4;
#pragma unroll
        for (int b = 0; b < 8; ++b)
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(A.out) + prow + 16 * b) =
                o.pk[tb][b];
    }
}

template <int STAGE, bool YF32>
__device__ __forceinline__ void pre_epilogue(const PreArgs &A, const f32x4 (&acc)[8][2], int nt,
                                             int tok0, int row0, int n_e, int wm, int wn,
                                             int lane, const int (&prow_tb)[2]) {
    const int g4 = lane >> 4;
    if (STAGE == 1) {
        // blocks b < 4: gate rows, b + 4: the matching up rows -> activation
        // columns nt*128 + 64wn + 16b + 4g4 + i; 32-column scale blocks j = b/2
        const int I = A.I;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int r = tok0 + 32 * wm + 16 * tb + (lane & 15);
            const bool ok = r < n_e;
            const size_t orow = (size_t)(row0 + (ok ? r : 0));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float a[2][4];
                float amax = 0.0f;
#pragma unroll
                for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int b = 2 * j + bb;
                        a[bb][i] = silu_mul_p(acc[b][tb][i], acc[b + 4][tb][i]);
                        amax = fmaxf(amax, fabsf(a[bb][i]));
                    }
                // the block's other 24 values sit in lanes lane ^ 16, ^ 32, ^ 48
                amax = fmaxf(amax, __shfl_xor(amax, 16));
                amax = fmaxf(amax, __shfl_xor(amax, 32));
                const int sb = split_scale_byte(amax);
                const float inv = split_inv_scale(sb);
                const int col0 = nt * 128 + 64 * wn + 32 * j;
#pragma unroll
                for (int bb = 0; bb < 2; ++bb) {
                    uint32_t h, l;
                    split_quad(a[bb], inv, h, l);
                    const size_t off = orow * I + col0 + 16 * bb + 4 * g4;
                    if (ok) {
                        *reinterpret_cast<uint32_t *>(A.ohi + off) = h;
                        *reinterpret_cast<uint32_t *>(A.olo + off) = l;
                    }
                }
                if (ok && g4 == 0) A.osc[orow * (I / 32) + col0 / 32] = (uint8_t)sb;
            }
        }
    } else {
        // all values packed before the first store (so no store's registers
        // are reused, and waited for, while others are still being written)
        uint2 pk[2][8];
        if (!YF32) {
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    pk[tb][b].x = pack_bf16x2(acc[b][tb][0], acc[b][tb][1]);
                    pk[tb][b].y = pack_bf16x2(acc[b][tb][2], acc[b][tb][3]);
                }
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int r = tok0 + 32 * wm + 16 * tb + (lane & 15);
            if (r >= n_e) continue;
            const size_t prow = (size_t)prow_tb[tb] * A.H + nt * 256 + 128 * wn + 4 * g4;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const size_t off = prow + 16 * b;
                if (YF32)
                    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(A.out) + off) = acc[b][tb];
                else
                    *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(A.out) + off) = pk[tb][b];
            }
        }
    }
}

template <int STAGE, bool YF32, int FMT>
__global__ __launch_bounds__(kPreThreads) void ffn_pre_kernel(PreArgs A) {
    __shared__ __attribute__((aligned(16))) PreStage<FMT> lds[kPreStages];
    constexpr int WB = wblock_bytes(FMT);
    const int tid = threadIdx.x, lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wv & 1, wn = wv >> 1;     // token half (32 tokens), weight half

    // total tile groups (nt_group consecutive weight tiles of one token tile),
    // then this workgroup's group (XCD-aware numbering), from the token-tile
    // map by scalar loads
    const MOE_CONST int32_t *map = as_scalar(A.tile_map);
    const int gpm = A.ntiles_w / A.nt_group;          // groups per token tile
    const long total = (long)map[0] * gpm;
    const long per = (total + 7) / 8;
    const long q = (long)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if ((long)(blockIdx.x >> 3) >= per || q >= total) return;
    const int m = (int)(q / gpm);
    const int nt = (int)(q - (long)m * gpm) * A.nt_group;   // first weight tile of the group
    const int md = map[1 + m];
    const int e = md & 0xFFFF, mt = md >> 16;

    const MOE_CONST int32_t *offs = as_scalar(A.offsets);
    // the shared expert (index E): rows T*k .. T*k + T - 1, token r = row r
    const bool sh = e == A.E;
    const int row0 = sh ? A.T * A.k : offs[e];
    const int n_e = sh ? A.T : offs[e + 1] - row0;
    const int tok0 = mt * kPreTok;
    // token blocks of this wavefront (rows tok0 + 32 wm + 16 tb ..) with rows of the expert
    const int left = n_e - tok0 - 32 * wm;
    const int nvb = left <= 0 ? 0 : left <= 16 ? 1 : 2;
    const MOE_CONST moe_expert_w *W = sh ? as_scalar(A.shared) : as_scalar(A.experts) + e;
    const uint8_t *wcodes = reinterpret_cast<const uint8_t *>(STAGE == 1 ? W->w13 : W->w2);
    const uint8_t *wscales = reinterpret_cast<const uint8_t *>(STAGE == 1 ? W->s13 : W->s2);
    const int nslab = A.K / 128;
    // stage 2: output rows (pair indices) of this lane's two tokens, loaded
    // before the copies so that the epilogue does not wait for them
    int prow_tb[2] = {0, 0};
    if (STAGE == 2) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int r = tok0 + 32 * wm + 16 * tb + (lane & 15);
            prow_tb[tb] = r >= n_e ? 0 : sh ? row0 + r : A.sorted_pair[row0 + r];
        }
    }

    PreSrc src;
    {
        auto token_row = [&](int r) -> long {   // operand row of tile row r
            r = r < n_e ? r : n_e - 1;             // rows past the expert's end repeat its last row
            if (STAGE == 1) return sh ? (long)r : (long)(A.sorted_pair[row0 + r] / A.k);
            return (long)(row0 + r);
        };
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            // token block wv, row 8u + lane/8; lane position lane%8 holds chunk pos ^ swizzle
            const int rb = 8 * u + (lane >> 3);
            const long row = token_row(tok0 + 16 * wv + rb);
            const int chunk = (lane & 7) ^ tok_swz(rb);
            src.thi[u] = A.bhi + row * A.K + 16 * chunk;
            src.tlo[u] = A.blo + row * A.K + 16 * chunk;
        }
        src.tsc = A.bsc + token_row(tok0 + lane) * (A.K / 32);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            src.wc[u] = wcodes + (size_t)pre_block<STAGE>(A, nt, 4 * wv + u) * nslab * WB +
                        16 * lane;
        src.ws = wscales + (size_t)pre_block<STAGE>(A, nt, lane >> 2) * nslab * 64 +
                 16 * (lane & 3);
    }

    f32x4 acc[8][2];
#pragma unroll
    for (int b = 0; b < 8; ++b)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[b][tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // weight tile nt + t starts (STAGE 1 ? 8 : 16) blocks after tile nt
    const size_t wstep = (size_t)(STAGE == 1 ? 8 : 16) * nslab * WB;
    // FP8: the matrix's fp32 scale multiplies the sums (the blocks use unit scales)
    const float gsc = FMT == MOE_W_FP8 ? *as_scalar(reinterpret_cast<const float *>(wscales)) : 1.0f;
    pre_issue<FMT>(lds[0], 0, wv, src, 0);
    // stage 2 with bf16 y: a tile's outputs are stored after the next tile's
    // first slab barrier (or at the end), not before it
    constexpr bool kDefer = STAGE == 2 && !YF32;
    PreOut pend;
    bool pending = false;
    // the tile group's loop, compiled for 2, 1 and 0 token blocks with rows
    // (a branch inside the slab loop instead made the kernels 1.6x slower)
    auto tiles = [&](auto nvb_c) {
        constexpr int NVB = decltype(nvb_c)::value;
        for (int t = 0; t < A.nt_group; ++t) {
            pre_mainloop<STAGE, FMT, NVB>(
                lds, acc, nslab, t * nslab, wv, wm, wn, lane, src, t * wstep, (t + 1) * wstep,
                t + 1 < A.nt_group, [&]() {
                    if (kDefer && pending) pre_store_y(A, pend, tok0, n_e, wm, wn, lane, prow_tb);
                });
            if (FMT == MOE_W_FP8) {
#pragma unroll
                for (int b = 0; b < 8; ++b)
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) acc[b][tb] *= gsc;
            }
            if (kDefer) {
                pre_pack_y(acc, nt + t, pend);
                pending = true;
            } else {
                pre_epilogue<STAGE, YF32>(A, acc, nt + t, tok0, row0, n_e, wm, wn, lane, prow_tb);
            }
#pragma unroll
            for (int b = 0; b < 8; ++b)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) acc[b][tb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    if (nvb == 2) tiles(std::integral_constant<int, 2>());
    else if (nvb == 1) tiles(std::integral_constant<int, 1>());
    else tiles(std::integral_constant<int, 0>());
    if (kDefer && pending) pre_store_y(A, pend, tok0, n_e, wm, wn, lane, prow_tb);
}


// Tiled path needs whole 128-row weight tiles in stage 1 (I % 128) and
// 256-row tiles in stage 2 (H % 256), and whole 128-column slabs.
bool ffn_prefill_supported(int fmt, int H, int I) {
    return (fmt == MOE_W_MXFP4 || fmt == MOE_W_FP8) && I % 128 == 0 && H % 256 == 0;
}

static size_t al256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace of the tiled path: the activation's two terms and scales
// [n_pairs][I] and the token rows' [T][H].
// (map[0] and at most n_pairs / 64 + E + 1 tiles: one partial tile per expert,
// the shared expert included)
static size_t tile_map_bytes(long n_pairs, int E) {
    return al256(((size_t)n_pairs / kPreTok + E + 3) * sizeof(int32_t));
}

size_t prefill_ws_bytes(long n_pairs, long T, int H, int I, int E) {
    return 2 * al256((size_t)n_pairs * I) + al256((size_t)n_pairs * I / 32) +
           2 * al256((size_t)T * H) + al256((size_t)T * H / 32) + tile_map_bytes(n_pairs, E);
}

template <int STAGE, bool YF32, int FMT>
static int launch_pre(hipStream_t s, PreArgs A, long n_pairs) {
    // n_pairs: rows over all experts of the launch (the shared expert's included)
    // weight tiles per workgroup: stage 2's short contraction (I / 128 slabs
    // per tile) runs several tiles per workgroup so the copy ring spans more
    // slabs (MOE_OPT_PRE_GROUP)
    int want = pre_group(STAGE);
    while (want > 1 && A.ntiles_w % want) --want;
    A.nt_group = want;
    // upper bound on token tiles: sum_e ceil(count_e / 64) <= n_pairs / 64 + E (+ 1 shared)
    const long mt_max = n_pairs / kPreTok + A.E + 1;
    const long tiles_max = mt_max * (A.ntiles_w / A.nt_group);
    const long grid = ((tiles_max + 7) / 8) * 8;
    if (grid > 0x7FFFFFFFL) return MOE_EUNSUPPORTED;
    MOE_LAUNCH(STAGE == 1 ? K_PRE_GATE_UP : K_PRE_DOWN, (ffn_pre_kernel<STAGE, YF32, FMT>), dim3((unsigned)grid),
                                 dim3(kPreThreads), 0, s, A);
    return check_launch();
}

int ffn_prefill(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
                const moe_expert_w *experts, const moe_expert_w *shared, int fmt, int T, int k,
                int H, int I, int E, void *y, int y_is_fp32, void *ws, hipStream_t s) {
    if (!ffn_prefill_supported(fmt, H, I)) return MOE_EUNSUPPORTED;
    // activation rows: the routed pairs, then the shared expert's T rows
    const long n = (long)T * k + (shared ? T : 0);
    uint8_t *p = reinterpret_cast<uint8_t *>(ws);
    uint8_t *ahi = p;
    uint8_t *alo = ahi + al256((size_t)n * I);
    uint8_t *asc = alo + al256((size_t)n * I);
    uint8_t *xhi = asc + al256((size_t)n * I / 32);
    uint8_t *xlo = xhi + al256((size_t)T * H);
    uint8_t *xsc = xlo + al256((size_t)T * H);
    int32_t *map = reinterpret_cast<int32_t *>(xsc + al256((size_t)T * H / 32));

    const long nblk = (long)T * H / 32;
    const long grid = (nblk * 4 + 255) / 256 + 1;   // four threads per block, + the tile-map workgroup
    if (grid > 0x7FFFFFFFL) return MOE_EUNSUPPORTED;
    MOE_LAUNCH(K_PRE_SPLIT, split_rows_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, nblk,
                                 xhi, xlo, xsc, offsets, E, shared ? T : 0, map);
    int rc = check_launch();
    if (rc) return rc;

    PreArgs a1{xhi, xlo, xsc, sorted_pair, offsets, experts, nullptr, ahi, alo, asc, map,
               shared, k, H, H, I, E, T, I / 128, 1};
    PreArgs a2{ahi, alo, asc, sorted_pair, offsets, experts, y, nullptr, nullptr, nullptr, map,
               shared, k, I, H, I, E, T, H / 256, 1};
    if (fmt == MOE_W_FP8) {
        rc = launch_pre<1, false, MOE_W_FP8>(s, a1, n);
        if (rc) return rc;
        return y_is_fp32 ? launch_pre<2, true, MOE_W_FP8>(s, a2, n)
                         : launch_pre<2, false, MOE_W_FP8>(s, a2, n);
    }
    rc = launch_pre<1, false, MOE_W_MXFP4>(s, a1, n);
    if (rc) return rc;
    return y_is_fp32 ? launch_pre<2, true, MOE_W_MXFP4>(s, a2, n)
                     : launch_pre<2, false, MOE_W_MXFP4>(s, a2, n);
}

}  // namespace moe
