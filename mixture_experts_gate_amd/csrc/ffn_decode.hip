// Decode-shaped grouped SwiGLU expert FFN: few tokens per expert, so the cost
// is streaming each touched expert's weights once from HBM.
//
// The pages place the cost of decoding a sparse MoE in expert-weight movement
// (winzheng.com page, "Why Now of All Times": only the routed experts'
// parameters take part per token). Every touched expert's weights are read
// exactly once, coalesced and non-temporal, decoded in registers (E2M1 x E8M0
// -> bf16 with the gfx950 scaled convert) and fed to bf16 matrix-core
// instructions whose other operand is the expert's tokens.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 as used here: lane l supplies row
// (l % 16) and K-chunk (l / 16) of A (8 consecutive K), column (l % 16) and
// the same K-chunk of B; it receives D[4 * (l / 16) + i][l % 16], i = 0..3.
// A lane loads 16 bytes = 32 FP4 weights = one scale block; its 4 groups of 8
// feed 4 MFMAs, and the token operand is loaded with the same K mapping, so
// the K order inside an MFMA is a consistent permutation on both sides.
//
// Work decomposition (both stages): a tile is NB 16-row blocks of one
// touched expert's matrix over the full contraction length K, for one block
// of at most 16 of the expert's rows; the KS wavefronts of a workgroup split
// K, and their partial sums meet in LDS (fixed order). Each workgroup owns a
// contiguous range of the U * tiles_per_expert tiles (U = row blocks of the
// experts with pairs, counted on the device), so the grid is fixed and no
// host round trip is needed. While a tile is being multiplied, the next
// tile's weights are already in flight; the token operand stays in registers
// while consecutive tiles belong to the same row block.
//   stage 1: blocks = 16 gate rows and the matching 16 up rows of W13 (K = H);
//            epilogue a = silu(g) * u -> act[sorted row][I] (bf16).
//   stage 2: blocks = 32 or 64 consecutive rows of W2 (K = I);
//            epilogue -> y[pair][H] (bf16 or fp32).
#include <math.h>

#include "common.hpp"

namespace moe {

constexpr int kPass = 16;     // tokens per MFMA pass (one 16-column block)
#ifndef MOE_DEC_DEPTH
#define MOE_DEC_DEPTH 2
#endif
#ifndef MOE_DEC_DEPTH2
#define MOE_DEC_DEPTH2 MOE_DEC_DEPTH
#endif
constexpr int kDepth = MOE_DEC_DEPTH;   // weight tiles held in registers (D - 1 in flight)
constexpr int kDepth2 = MOE_DEC_DEPTH2; // the same for stage 2

// silu(g) * u with the hardware reciprocal (about 1 ulp) in place of a
// correctly rounded division
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Position of a tile: active expert a, tile rt within it; advanced by a
// fixed stride of (sa, srt) tiles without divisions.
struct TilePos {
    int a, rt;
};

__device__ __forceinline__ TilePos advance(TilePos p, int sa, int srt, int nrt) {
    p.a += sa;
    p.rt += srt;
    if (p.rt >= nrt) {
        p.rt -= nrt;
        p.a += 1;
    }
    return p;
}

// One lane's weights for one 32-element K block of one row.
template <int FMT>
struct WFrag;

template <>
struct WFrag<MOE_W_MXFP4> {
    u32x4 q;
    uint32_t s;
    // Opaque to the optimiser: keeps the decode next to its use instead of
    // hoisting every decoded fragment out of the token-pass loop.
    __device__ __forceinline__ void pin() { asm volatile("" : "+v"(q), "+v"(s)); }
    // kernel layout: block `chunk` = (row block, 128-column slab); lane l's
    // 16 code bytes and scale byte sit at lane-contiguous positions. Always
    // issued; !ok loads zeros (codes 0 decode to 0 under any scale).
    __device__ __forceinline__ void load_block(buf_rsrc codes, buf_rsrc scales, uint32_t chunk,
                                               int lane, bool ok) {
        q = buf_load_nt16(codes, ok ? chunk * 1024u + lane * 16 : kBufOff);
        s = buf_load_u8(scales, ok ? chunk * 64u + lane : kBufOff);
    }
    __device__ __forceinline__ bf16x8 get(int j) const { return dequant8_fp4(q[j], e8m0_to_f32(s)); }
};

// NVFP4: the lane's 32 codes span two 16-element blocks (dwords 0-1 and 2-3),
// each with an E4M3 scale. The convert applies only a power of two, so a
// block scale v is split into 2^floor(log2 v) (in the convert, to fp16) and
// its mantissa factor in [1, 2) (one packed fp16 multiply per two elements).
// code x v has at most 6 significant bits and lies in [2^-10, 2880], so it is
// exact in fp16; these weights run through the fp16 matrix instruction (the
// token operand is carried in fp16 too). The matrix's fp32 scale multiplies
// the sums instead (epilogue).
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

template <>
struct WFrag<MOE_W_NVFP4> {
    u32x4 q;
    uint32_t s;     // two E4M3 block-scale bytes
    __device__ __forceinline__ void pin() { asm volatile("" : "+v"(q), "+v"(s)); }
    __device__ __forceinline__ void load_block(buf_rsrc codes, buf_rsrc scales, uint32_t chunk,
                                               int lane, bool ok) {
        q = buf_load_nt16(codes, ok ? chunk * 1024u + lane * 16 : kBufOff);
        s = __builtin_amdgcn_raw_buffer_load_b16(scales, ok ? chunk * 128u + lane * 2 : kBufOff,
                                                 0, kBufNt);
    }
    __device__ __forceinline__ f16x8 get(int j) const {
        const uint32_t sb = (j >> 1) ? (s >> 8) : s;
        const float v = __builtin_amdgcn_cvt_f32_fp8((int)sb, 0);         // block scale
        const uint32_t b = __float_as_uint(v);
        const float p2 = __uint_as_float(b & 0x7F800000u);
        const _Float16 mh =
            v == 0.0f ? (_Float16)0.0f : (_Float16)__uint_as_float((b & 0x007FFFFFu) | 0x3F800000u);
        const f16x2 m2 = {mh, mh};
        const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q[j], p2, 0) * m2;
        const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q[j], p2, 1) * m2;
        const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q[j], p2, 2) * m2;
        const f16x2 e = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q[j], p2, 3) * m2;
        f16x8 r = {a[0], a[1], c[0], c[1], d[0], d[1], e[0], e[1]};
        return r;
    }
};

// FP8 E4M3: 32 one-byte codes per lane (two 16-byte loads); codes enter the
// products exactly (scale 1) and the matrix's fp32 scale multiplies the sums.
template <>
struct WFrag<MOE_W_FP8> {
    u32x4 q[2];
    __device__ __forceinline__ void pin() { asm volatile("" : "+v"(q[0]), "+v"(q[1])); }
    __device__ __forceinline__ void load_block(buf_rsrc codes, buf_rsrc, uint32_t chunk, int lane,
                                               bool ok) {
        const uint32_t o = ok ? chunk * 2048u + lane * 32 : kBufOff;
        q[0] = buf_load_nt16(codes, o);
        q[1] = buf_load_nt16(codes, o + 16);
    }
    __device__ __forceinline__ bf16x8 get(int j) const {
        const u32x4 &w = q[j >> 1];
        const uint32_t lo = w[(j & 1) * 2], hi = w[(j & 1) * 2 + 1];
        const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
        const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
        const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
        const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
        bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
        return r;
    }
};

// Formats whose kernel layout is the 16 x 128 block tiling.
constexpr bool blocked_fmt(int fmt) {
    return fmt == MOE_W_MXFP4 || fmt == MOE_W_NVFP4 || fmt == MOE_W_FP8;
}
// Formats with one fp32 scale per matrix, applied to the sums.
constexpr bool tensor_scaled(int fmt) { return fmt == MOE_W_NVFP4 || fmt == MOE_W_FP8; }
// Formats whose products run in fp16 (weights, tokens and the activation).
constexpr bool f16_path(int fmt) { return fmt == MOE_W_NVFP4; }

// 8 bf16 (one u32x4) -> 8 fp16, in place; exact for magnitudes in
// [2^-14, 65504] (fp16 keeps more significand bits than bf16).
__device__ __forceinline__ void bf16x8_to_f16(u32x4 &v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xFFFF0000u);
        const f16x2 h = {(_Float16)lo, (_Float16)hi};
        v[i] = __builtin_bit_cast(uint32_t, h);
    }
}

template <>
struct WFrag<MOE_W_BF16> {
    u32x4 q[4];
    __device__ __forceinline__ void pin() { asm volatile("" : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3])); }
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

// The shared expert of a launch that carries one, as active experts with
// index E after the routed ones: its T token rows in blocks of one token pass
// (16 rows), each one more active entry, so the blocks read the same weights
// close together in time (mostly from cache). Token t's activation and output
// row is base + t, base = T*k. A second kernel argument, so that launches
// without it keep the argument layout (and scalar registers) they had.
struct ShArgs {
    const moe_expert_w *shared;
    int T, base;
};

// Inclusive prefix sum over the wavefront: within rows of 16 lanes by DPP
// row shifts (lanes before a row's start read 0), then the totals of the
// rows before this lane's, by lane reads.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    const int t0 = __builtin_amdgcn_readlane(v, 15);
    const int t1 = __builtin_amdgcn_readlane(v, 31);
    const int t2 = __builtin_amdgcn_readlane(v, 47);
    const int r = lane_id() >> 4;
    return v + (r >= 1 ? t0 : 0) + (r >= 2 ? t1 : 0) + (r >= 3 ? t2 : 0);
}

// Active experts in blocks of one token pass: an expert that received r > 0
// pairs takes ceil(r / 16) consecutive active entries, each with at most 16
// rows, so every tile has one token pass and the launch keeps its contiguous
// tile order whatever the popularity skew (a hot expert's blocks sit side by
// side and read the same weights close together in time). For group i of 64
// experts, lane l holds the inclusive count of blocks of experts 64i ..
// 64i + l (a wavefront scan, from one round of loads); a lookup is a ballot
// and a lane read. With a shared expert its ceil(T/16) blocks come last, with
// expert index E. Requires E <= 512.
// A gate/up launch may also take the routing ids instead of the permutation
// and derive what it needs itself (moe_permute_ffn_combine), so that no
// permutation launch runs before it: every wavefront of a tile workgroup
// counts the ids per expert in its own LDS region (no barrier: one
// wavefront's LDS operations run in order) for the offsets, and finds a
// block's pairs, the occurrences j*16 .. j*16+15 of its expert in pair
// order, with one ballot per 64-pair chunk. One more workgroup (index 0,
// dispatched first) ranks all pairs, the stable counting sort of
// moe_permute, and writes the permutation out for the down projection and
// the combine. Per wavefront: offsets [E + 1], running bases [E], sorted
// pairs [n] (used by workgroup 0 only).
constexpr int kIdsMaxPairs = 512;       // pairs (T * k) of such a launch
constexpr size_t kLdsPerCu = 160 * 1024;
constexpr int kIdsMaxE = 256;           // experts: ids fit 8 bits
constexpr int kIdsChunks = kIdsMaxPairs / kWave;
__host__ __device__ constexpr int ids_wave_ints(int E, int n) { return (2 * E + 1 + n + 3) & ~3; }

// Rank of this lane's value e among the lanes before it with the same e
// (lanes with !valid take no part), by one ballot per bit of e (a
// multisplit); *same = lanes with this lane's e.
template <int NBITS>
__device__ __forceinline__ int wave_rank_bits(bool valid, int e, int *same) {
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < NBITS; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    *same = __popcll(m);
    return __popcll(m & lanemask_lt());
}

// Position of the k-th (0-based) set bit of b (k < popcount(b)).
__device__ __forceinline__ int nth_bit(uint64_t b, int k) {
    const uint32_t lo = (uint32_t)b;
    const int plo = __popc(lo);
    const bool hi = k >= plo;
    uint32_t w = hi ? (uint32_t)(b >> 32) : lo;
    int pos = hi ? 32 : 0;
    k = hi ? k - plo : k;
#pragma unroll
    for (int sh = 16; sh >= 1; sh >>= 1) {
        const int pl = __popc(w & ((1u << sh) - 1u));
        const bool up = k >= pl;
        k = up ? k - pl : k;
        w = up ? w >> sh : w;
        pos += up ? sh : 0;
    }
    return pos;
}

struct ActiveSet {
    int gtot[8];             // blocks of expert group i (wavefront-uniform)
    int incl[8];             // lane l: blocks of experts 64i .. 64i + l
    int count;               // blocks, the shared expert's included
    int routed;              // blocks of routed experts
    const moe_expert_w *sh_w;  // shared expert's weights and tokens (SH launches)
    int sh_T;
    // launches from the routing ids: this wavefront's permutation in LDS
    int *loff;               // [E + 1] offsets, then [E] running bases
    int *lsrt;               // [n] sorted pair indices
    int idv[kIdsChunks];     // lane l: id of pair 64c + l (-1: none, or outside [0, E))

    // From the routing ids (n <= kIdsMaxPairs pairs, E <= kIdsMaxE): the
    // counts and offsets; the ranks follow in rank_ids. wl: ids_wave_ints(E, n)
    // ints of LDS for this wavefront alone.
    template <bool SH>
    __device__ __forceinline__ void init_ids(const int32_t *__restrict__ ids, int n, int E,
                                             const ShArgs &S, int *wl, int *ids_wg) {
        const int lane = lane_id();
        loff = wl;
        int *cnt = wl + E + 1;
        lsrt = wl + 2 * E + 1;
        for (int e = lane; e < E; e += kWave) cnt[e] = 0;
        // the workgroup's wavefronts load the chunks in turn (lanes past n
        // read the last id again and drop it) into the workgroup's copy
        // (ids_wg, kIdsMaxPairs ints), and each then reads all of them
        const int wv = threadIdx.x / kWave, nw = blockDim.x / kWave;
        for (int c = wv; c < kIdsChunks; c += nw) {
            if (c * kWave < n) {
                const int p = c * kWave + lane;
                const int v = ids[min(p, n - 1)];
                ids_wg[p] = p < n && v >= 0 && v < E ? v : -1;
            }
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < kIdsChunks; ++c) idv[c] = c * kWave < n ? ids_wg[c * kWave + lane] : -1;
#pragma unroll
        for (int c = 0; c < kIdsChunks; ++c)
            if (idv[c] >= 0) atomicAdd(&cnt[idv[c]], 1);
        // per group of 64 experts: offsets (exclusive scan of the counts) and
        // blocks (as init)
        count = 0;
        int base = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            incl[i] = 0;
            gtot[i] = 0;
            if (i * kWave < E) {
                const int e = i * kWave + lane;
                const int ce = e < E ? cnt[e] : 0;
                const int ic = wave_incl_scan(ce);
                if (e < E) {
                    loff[e] = base + ic - ce;
                    cnt[e] = base + ic - ce;
                }
                base += __builtin_amdgcn_readlane(ic, kWave - 1);
                incl[i] = wave_incl_scan((ce + kPass - 1) / kPass);
                gtot[i] = __builtin_amdgcn_readlane(incl[i], kWave - 1);
            }
            count += gtot[i];
        }
        if (lane == 0) loff[E] = base;
        routed = count;
        if constexpr (SH) {
            count += (S.T + kPass - 1) / kPass;
            sh_w = S.shared;
            sh_T = S.T;
        }
    }
    // Pair index of occurrence q (in pair order) of expert e (q past e's
    // pairs: 0), by one ballot per chunk, the chunk holding q chosen by
    // selects against the chunks' running counts, and one bit search. No
    // branches: a branch here, inside the tile loop, made the compiler's
    // waits before the products also wait for part of the weight prefetch.
    __device__ __forceinline__ int pair_of(int e, int q) const {
        uint64_t bm = 0;
        int before = 0, base = 0, cc = 0;
#pragma unroll
        for (int c = 0; c < kIdsChunks; ++c) {
            const uint64_t b = __ballot(idv[c] == e);
            const bool ge = q >= before;        // chunk c starts at or before q
            bm = ge ? b : bm;
            base = ge ? before : base;
            cc = ge ? c : cc;
            before += __popcll(b);
        }
        const bool ok = q < before;
        return ok ? cc * kWave + nth_bit(bm, ok ? q - base : 0) : 0;
    }
    // Stable ranks: pair p of expert e goes to lsrt[offsets[e] + (pairs of e
    // before p)], chunk by chunk in pair order.
    __device__ __forceinline__ void rank_ids(int n, int E) {
        const int lane = lane_id();
        int *cnt = loff + E + 1;
#pragma unroll
        for (int c = 0; c < kIdsChunks; ++c) {
            if (c * kWave < n) {
                const bool valid = idv[c] >= 0;
                int same;
                const int r = wave_rank_bits<8>(valid, idv[c], &same);
                if (valid) {
                    const int b = cnt[idv[c]];
                    lsrt[b + r] = c * kWave + lane;
                    if (r == 0) cnt[idv[c]] = b + same;
                }
            }
        }
    }
    template <bool SH>
    __device__ __forceinline__ void init(const int32_t *__restrict__ offsets, int E,
                                         const ShArgs &S) {
        const int lane = lane_id();
        // all loads first (experts past E read offsets[E] twice: no rows),
        // so that one wait covers them; groups wholly past E are skipped
        int o0[8], o1[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            o0[i] = o1[i] = 0;
            if (i * kWave < E) {
                const int e = min(i * kWave + lane, E);
                o0[i] = offsets[e];
                o1[i] = offsets[min(e + 1, E)];
            }
        }
        count = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            incl[i] = 0;
            gtot[i] = 0;
            if (i * kWave < E) {
                incl[i] = wave_incl_scan((o1[i] - o0[i] + kPass - 1) / kPass);
                gtot[i] = __builtin_amdgcn_readlane(incl[i], kWave - 1);
            }
            count += gtot[i];
        }
        routed = count;
        if constexpr (SH) {
            count += (S.T + kPass - 1) / kPass;
            sh_w = S.shared;
            sh_T = S.T;
        }
    }
    // expert of the a-th block (a < count; a shared-expert block: E) and the
    // block's index j within that expert
    template <bool SH>
    __device__ __forceinline__ int nth(int a, int E, int &j) const {
        if constexpr (SH) {
            if (a >= routed) {
                j = a - routed;
                return E;
            }
        }
        // the group holding block a, found with constant indices only (a
        // dynamically indexed array would live in scratch memory, and its
        // load's wait would also drain the weight prefetch in flight)
        int g = 0, ai = a, inc = incl[0], before = 0;
        bool found = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool here = !found && a - before < gtot[i];
            g = here ? i : g;
            ai = here ? a - before : ai;
            inc = here ? incl[i] : inc;
            found = found || here;
            before += gtot[i];
        }
        const uint64_t m = __ballot(inc > ai);
        const int l = __ffsll((long long)m) - 1;
        j = ai - (l ? __builtin_amdgcn_readlane(inc, l - 1) : 0);
        return g * kWave + l;
    }
};

// Routing ids of a gate/up launch that derives the permutation (init_ids);
// the permutation's offsets and sorted pairs go to DecArgs' offsets and
// sorted_pair, which are outputs then.
struct IdsArgs {
    const int32_t *ids;             // [n] expert ids of the pairs (topk_ids)
    int32_t *pair_row;              // [n] output: sorted position of each pair
    int n;
};

struct DecArgs {
    const uint16_t *src;            // B-operand rows: x [T][H] (stage 1) or act [T*k][I] (stage 2)
    const int32_t *sorted_pair;
    const int32_t *offsets;
    const moe_expert_w *experts;
    void *out;                      // act (stage 1) or y (stage 2)
    int k, K, H, I, E, nrt;         // nrt: tiles per expert
    // weighted split of the tiles over the workgroups (see split_start)
    int slot_size;                  // workgroups per dispatch slot (compute units)
    float w_slot, w_pos;
};

// Share of the tiles before workgroup b when workgroup i carries weight
// 1 - w_slot * (i / C) - w_pos * (i % C) / C (C = slot_size): a persistent
// grid is dispatched one workgroup per compute unit at a time, and a
// workgroup dispatched later (a later slot on its compute unit, or later
// within a slot) receives its first weights later, because the start-up
// burst of requests is served roughly in issue order; with equal shares it
// also finishes later, by the same offset, while the early ones idle.
// Returns the weight sum over workgroups 0 .. b-1.
__device__ __forceinline__ float split_prefix(int b, int C, float ws, float wp) {
    const int s = b / C, r = b - s * C;
    const float full = (float)s * ((float)C - wp * (float)(C - 1) * 0.5f) -
                       ws * (float)C * ((float)s * (float)(s - 1) * 0.5f);
    const float part = (float)r * (1.0f - ws * (float)s) -
                       wp * ((float)r * (float)(r - 1) * 0.5f) / (float)C;
    return full + part;
}

__device__ __forceinline__ int split_start(int b, int G, int total, const DecArgs &A) {
    if (b >= G) return total;
    const float f = split_prefix(b, A.slot_size, A.w_slot, A.w_pos) /
                    split_prefix(G, A.slot_size, A.w_slot, A.w_pos);
    const int t = (int)((float)total * f);
    return t < total ? t : total;
}


// Expert-level state of the tile being processed (wavefront-uniform: read
// with scalar loads, so fetching it never waits for the weights in flight).
// the matrix's fp32 scale, a member only for the formats that have one
template <bool HAS>
struct TensorScale {
    float g;
};
template <>
struct TensorScale<false> {};

template <int FMT>
struct ExpertState : TensorScale<tensor_scaled(FMT)> {
    int a, e, row0, n_e;
    const uint8_t *w, *s;           // matrix base (W13 or W2) and its scales
    buf_rsrc wr, sr;                // the same as ranged buffer resources (block formats)
};

// SH: the launch carries the shared expert (compiled out otherwise). Only its
// weights and token count stay in registers (the gate/up kernels run at the
// scalar-register limit); block size and row base are derived where used.
template <int STAGE, int FMT, bool SH, bool IDS = false>
__device__ __forceinline__ void expert_state(const DecArgs &A, const ShArgs &S,
                                             const ActiveSet &act, int a, ExpertState<FMT> &st) {
    st.a = a;
    int j;                                    // block of the expert
    st.e = act.template nth<SH>(a, A.E, j);
    const bool sh = SH && st.e == A.E;        // a block of the shared expert's tokens
    int o_lo, o_hi;                           // offsets[e], offsets[e + 1]
    if constexpr (IDS) {
        // from this wavefront's LDS copy (uniform address; e == E reads
        // past the offsets, unused)
        o_lo = __builtin_amdgcn_readfirstlane(act.loff[st.e]);
        o_hi = __builtin_amdgcn_readfirstlane(act.loff[st.e + 1]);
    } else {
        const MOE_CONST int32_t *off = as_scalar(A.offsets);
        o_lo = off[st.e];
        o_hi = off[st.e + 1];
    }
    st.row0 = (sh ? act.sh_T * A.k : o_lo) + j * kPass;
    st.n_e = min(kPass, (sh ? act.sh_T * (A.k + 1) : o_hi) - st.row0);
    const MOE_CONST moe_expert_w *W = sh ? as_scalar(act.sh_w) : as_scalar(A.experts) + st.e;
    st.w = reinterpret_cast<const uint8_t *>(STAGE == 1 ? W->w13 : W->w2);
    st.s = reinterpret_cast<const uint8_t *>(STAGE == 1 ? W->s13 : W->s2);
    const uint32_t elems = (uint32_t)(STAGE == 1 ? 2 * A.I : A.H) * (uint32_t)A.K;
    st.wr = make_rsrc(st.w, FMT == MOE_W_FP8 ? elems : elems / 2);
    st.sr = make_rsrc(st.s, FMT == MOE_W_NVFP4 ? elems / 16 : elems / 32);
    if constexpr (FMT == MOE_W_NVFP4)
        st.g = *as_scalar(reinterpret_cast<const float *>(st.s + elems / 16));
    if constexpr (FMT == MOE_W_FP8) st.g = *as_scalar(reinterpret_cast<const float *>(st.s));
}

// 16-row block index (within the stage's matrix) of block b of tile rt.
// Stage 1: the first NB/2 blocks are gate rows, the last NB/2 the matching up rows.
template <int STAGE, int NB>
__device__ __forceinline__ long tile_block(const DecArgs &A, int rt, int b) {
    if (STAGE == 1) {
        constexpr int H2 = NB / 2;
        return b < H2 ? (long)rt * H2 + b : (long)A.I / 16 + (long)rt * H2 + (b - H2);
    }
    return (long)rt * NB + b;
}

// FULL: the KS wavefronts x SPW slabs cover the K slabs exactly (no bounds checks).
// `on` = false issues the same loads switched off (MXFP4; see buf_rsrc).
template <int FMT, int STAGE, int SPW, int NB, bool FULL>
__device__ __forceinline__ void load_tile(const DecArgs &A, const ExpertState<FMT> &st, int rt, int wv,
                                          int lane, WFrag<FMT> (&f)[SPW][NB], bool on = true) {
    if constexpr (blocked_fmt(FMT)) {
        const int nslab = A.K / 128;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const long rb = tile_block<STAGE, NB>(A, rt, b);
#pragma unroll
            for (int s = 0; s < SPW; ++s) {
                const int slab = wv * SPW + s;
                f[s][b].load_block(st.wr, st.sr, (uint32_t)(rb * nslab + slab), lane,
                                   on && (FULL || slab < nslab));
            }
        }
    } else {
        if (!on) return;
        const int nblk = A.K / 32, m = lane & 15, c = lane >> 4;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const long r = tile_block<STAGE, NB>(A, rt, b) * 16 + m;
            const uint8_t *cr = wrow<FMT>(st.w, r, A.K);
#pragma unroll
            for (int s = 0; s < SPW; ++s) {
                const int kb = (wv * SPW + s) * 4 + c;
                f[s][b].load(cr, nullptr, kb, kb < nblk);
            }
        }
    }
}

// Token operand of pass p (rows p*16 .. p*16+15 of the expert), K slabs of
// this wavefront; for stage 2 also the pair index each row's output goes to.
template <int STAGE, int SPW, bool SH, bool IDS, class ES>
__device__ __forceinline__ void load_tokens(const DecArgs &A, const ShArgs &S, const ES &st,
                                            int p, int wv, int m, int c, u32x4 (&xr)[SPW][4],
                                            int &pidx, const ActiveSet &act) {
    const int nblk = A.K / 32;
    const int r = p * kPass + m;
    const bool has = r < st.n_e;
    const uint16_t *row;
    // shared-expert block: row r is token row0 - base + r; its output row is row0 + r
    const bool sh = SH && st.e == A.E;
    if (STAGE == 1 && IDS) {
        // lane m's pair: occurrence (row - offsets[e]) of the expert among the
        // ids (rows past the block give pair 0, not loaded)
        const int q = st.row0 - __builtin_amdgcn_readfirstlane(act.loff[st.e]) + r;
        const int pair = act.pair_of(st.e, q);
        row = A.src + (size_t)(sh ? st.row0 - S.T * A.k + r : pair / A.k) * A.K;
    } else if (STAGE == 1) {
        // the pass's 16 pair indices by scalar loads; lane m takes the m-th.
        // (A shared-expert block reads the first entries instead, in bounds
        // since p * 16 + i < n_e <= T <= T*k, and takes its token: a select,
        // no branch around the loads.)
        const MOE_CONST int32_t *sp = as_scalar(A.sorted_pair) + (sh ? 0 : st.row0 + p * kPass);
        int pair = 0;
#pragma unroll
        for (int i = 0; i < kPass; ++i)
            if (p * kPass + i < st.n_e) pair = m == i ? sp[i] : pair;
        row = A.src + (size_t)(sh ? st.row0 - S.T * A.k + r : pair / A.k) * A.K;
    } else {
        row = A.src + (size_t)(st.row0 + (has ? r : 0)) * A.K;
        pidx = !has ? 0 : sh ? st.row0 + r : A.sorted_pair[st.row0 + r];
    }
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
        const int kb = (wv * SPW + s) * 4 + c;
        const bool ld = has && kb < nblk;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            xr[s][j] = ld ? load16(row + kb * 32 + j * 8) : u32x4{0, 0, 0, 0};
    }
}

// One tile: token operand if the expert changed, prefetch of the next tile's
// weights into `wn`, multiply from `wc`, K-split reduction, epilogue.
template <int FMT, int STAGE, int SPW, int KS, int NB, bool YF32, bool FULL, int D, bool SH,
          bool IDS, bool COH = false>
__device__ __forceinline__ void dec_step(const DecArgs &A, const ShArgs &S, const ActiveSet &act,
                                         float (&red)[2][KS > 1 ? KS - 1 : 1][NB][4][kWave],
                                         WFrag<FMT> (&wc)[SPW][NB], WFrag<FMT> (&wn)[SPW][NB],
                                         u32x4 (&xr)[SPW][4], const ExpertState<FMT> &cur,
                                         const ExpertState<FMT> &prev, ExpertState<FMT> &nxt,
                                         int &pidx, int &x_key, bool &x_raw, int &buf, int rt,
                                         TilePos pn, bool pf, int lane, int wv, int m, int c) {

        // token operand for the first pass of this tile (loaded before the next
        // prefetch, so that waiting for it does not wait for the prefetched weights).
        // x_key: the active expert whose first pass the registers hold, or -1
        if (x_key != cur.a) {
            load_tokens<STAGE, SPW, SH, IDS>(A, S, cur, 0, wv, m, c, xr, pidx, act);
            x_key = cur.a;
            x_raw = true;
        }
        // prefetch the tile D - 1 steps ahead (position pn, present if pf);
        // `prev` holds the state of the tile before it. Issued, switched off,
        // also past the end (see buf_rsrc).
        const int an = pf ? pn.a : prev.a;
        if (an != prev.a) expert_state<STAGE, FMT, SH, IDS>(A, S, act, an, nxt);
        else nxt = prev;
        load_tile<FMT, STAGE, SPW, NB, FULL>(A, nxt, pf ? pn.rt : 0, wv, lane, wn, pf);
        for (int p = 0; p * kPass < cur.n_e; ++p) {
            if (p > 0) {   // more than 16 tokens: next 16 of this expert
                load_tokens<STAGE, SPW, SH, IDS>(A, S, cur, p, wv, m, c, xr, pidx, act);
                x_key = -1;     // a later pass: the next tile reloads its first
                x_raw = true;
            }
            // fp16 products: bf16 tokens (stage 1) are converted once per load
            // (after the prefetch was issued, so the wait for them leaves it in flight)
            if constexpr (f16_path(FMT) && STAGE == 1) {
                if (x_raw) {
#pragma unroll
                    for (int s = 0; s < SPW; ++s)
#pragma unroll
                        for (int j = 0; j < 4; ++j) bf16x8_to_f16(xr[s][j]);
                    x_raw = false;
                }
            }
            f32x4 acc[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < SPW; ++s)
#pragma unroll
                for (int b = 0; b < NB; ++b) wc[s][b].pin();
#pragma unroll
            for (int s = 0; s < SPW; ++s)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (f16_path(FMT)) {
                        const f16x8 hx = __builtin_bit_cast(f16x8, xr[s][j]);
#pragma unroll
                        for (int b = 0; b < NB; ++b)
                            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wc[s][b].get(j), hx,
                                                                           acc[b], 0, 0, 0);
                    } else {
                        const bf16x8 bx = as_bf16x8(xr[s][j]);
#pragma unroll
                        for (int b = 0; b < NB; ++b)
                            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wc[s][b].get(j), bx,
                                                                            acc[b], 0, 0, 0);
                    }
                }
            // partial sums of the K split meet in LDS (double-buffered: one barrier per pass)
            if (KS > 1) {
                if (wv > 0) {
#pragma unroll
                    for (int b = 0; b < NB; ++b)
#pragma unroll
                        for (int i = 0; i < 4; ++i) red[buf][wv - 1][b][i][lane] = acc[b][i];
                }
                __syncthreads();
            }
            if (wv == 0) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int w = 0; w < KS - 1; ++w) acc[b][i] += red[buf][w][b][i][lane];
                if constexpr (tensor_scaled(FMT)) {
#pragma unroll
                    for (int b = 0; b < NB; ++b)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[b][i] *= cur.g;
                }
                const int r = p * kPass + m;
                if (r < cur.n_e) {
                    if (STAGE == 1) {
                        constexpr int H2 = NB / 2;
                        uint16_t *actp = reinterpret_cast<uint16_t *>(A.out) + (size_t)(cur.row0 + r) * A.I;
#pragma unroll
                        for (int b = 0; b < H2; ++b) {
                            uint2 pk;
                            // the activation in the stage-2 operand type (bf16, or fp16)
                            auto pack2 = [](float lo, float hi) -> uint32_t {
                                if constexpr (f16_path(FMT)) {
                                    const f16x2 h = {(_Float16)lo, (_Float16)hi};
                                    return __builtin_bit_cast(uint32_t, h);
                                } else {
                                    return pack_bf16x2(lo, hi);
                                }
                            };
                            pk.x = pack2(silu_mul(acc[b][0], acc[b + H2][0]),
                                         silu_mul(acc[b][1], acc[b + H2][1]));
                            pk.y = pack2(silu_mul(acc[b][2], acc[b + H2][2]),
                                         silu_mul(acc[b][3], acc[b + H2][3]));
                            uint16_t *ap = actp + (rt * H2 + b) * 16 + 4 * c;
                            if constexpr (COH) {
                                // written through to the device's coherence point
                                // (read in the same launch by other workgroups)
                                __hip_atomic_store(reinterpret_cast<uint64_t *>(ap),
                                                   (uint64_t)pk.x | ((uint64_t)pk.y << 32),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            } else {
                                *reinterpret_cast<uint2 *>(ap) = pk;
                            }
                        }
                    } else {
                        const size_t prow = (size_t)pidx * A.H;
#pragma unroll
                        for (int b = 0; b < NB; ++b) {
                            const size_t off = prow + (size_t)(rt * NB + b) * 16 + 4 * c;
                            if (YF32) {
                                *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(A.out) + off) = acc[b];
                            } else {
                                uint2 pk;
                                pk.x = pack_bf16x2(acc[b][0], acc[b][1]);
                                pk.y = pack_bf16x2(acc[b][2], acc[b][3]);
                                *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(A.out) + off) = pk;
                            }
                        }
                    }
                }
            }
            buf ^= 1;
        }
}

// Workgroup 0 of a launch from the routing ids writes the permutation out
// (offsets, sorted pairs and each pair's sorted position, as moe_permute).
__device__ __forceinline__ void write_perm(const DecArgs &A, const IdsArgs &I,
                                           const ActiveSet &act) {
    const int lane = lane_id();
    int32_t *offsets = const_cast<int32_t *>(A.offsets);
    int32_t *sorted = const_cast<int32_t *>(A.sorted_pair);
    for (int e = lane; e <= A.E; e += kWave) offsets[e] = act.loff[e];
    const int nv = act.loff[A.E];
    for (int q = lane; q < nv; q += kWave) {
        const int pair = act.lsrt[q];
        sorted[q] = pair;
        I.pair_row[pair] = q;
    }
}

template <int FMT, int STAGE, int SPW, int KS, int NB, bool YF32, bool FULL, bool SH, bool IDS,
          bool COH = false>
__device__ __forceinline__ void dec_tiles(const DecArgs &A, const ShArgs &S, const ActiveSet &act,
                                          float (&red)[2][KS > 1 ? KS - 1 : 1][NB][4][kWave],
                                          int t0, int n);

template <int FMT, int STAGE, int SPW, int KS, int NB, bool YF32, bool FULL, bool SH, bool IDS>
__device__ __forceinline__ void ffn_dec_body(const DecArgs &A, const ShArgs &S, const IdsArgs &I,
                                             float (&red)[2][KS > 1 ? KS - 1 : 1][NB][4][kWave],
                                             int *ids_lds) {
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wavefront-uniform
    ActiveSet act;
    if constexpr (IDS) {
        act.template init_ids<SH>(I.ids, I.n, A.E, S, ids_lds + wv * ids_wave_ints(A.E, I.n),
                                  ids_lds + KS * ids_wave_ints(A.E, I.n));
        if (blockIdx.x == 0) {
            // the permutation workgroup: one wavefront ranks and writes
            if (wv == 0) {
                act.rank_ids(I.n, A.E);
                write_perm(A, I, act);
            }
            return;
        }
    } else {
        act.template init<SH>(A.offsets, A.E, S);
    }
    // Tiles are block-major (a block: up to 16 rows of one expert). Workgroups
    // take contiguous ranges, which keep a block's token operand in registers
    // across its tiles; every tile costs one token pass, so equal ranges are
    // balanced. (Launches from the ids: tile workgroups 1 .. grid - 1.)
    const int wb = IDS ? blockIdx.x - 1 : blockIdx.x, wg = IDS ? gridDim.x - 1 : gridDim.x;
    const int total = act.count * A.nrt;
    const int t0 = split_start(wb, wg, total, A);
    const int n = split_start(wb + 1, wg, total, A) - t0;
    if (n <= 0) return;
    dec_tiles<FMT, STAGE, SPW, KS, NB, YF32, FULL, SH, IDS>(A, S, act, red, t0, n);
}

// Tiles t0 .. t0 + n - 1 (n > 0) of a launch, by every wavefront of the
// workgroup (the K-split reduction has workgroup barriers). COH: stage-1
// activation stores written through to the coherence point.
template <int FMT, int STAGE, int SPW, int KS, int NB, bool YF32, bool FULL, bool SH, bool IDS,
          bool COH>
__device__ __forceinline__ void dec_tiles(const DecArgs &A, const ShArgs &S, const ActiveSet &act,
                                          float (&red)[2][KS > 1 ? KS - 1 : 1][NB][4][kWave],
                                          int t0, int n) {
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wavefront-uniform
    const int m = lane & 15, c = lane >> 4;
    const int sa = 0, srt = 1;

    // D register buffers used in turn: tile i computes from one while the
    // weights of tiles i+1 .. i+D-1 are in flight into the others (no copies
    // between them, so nothing waits for a prefetch before it is needed).
    // Slots past the end repeat the last tile's position and load nothing.
    constexpr int D = STAGE == 2 ? kDepth2 : kDepth;
    ExpertState<FMT> es[D];
    TilePos pos[D];
    WFrag<FMT> wr[D][SPW][NB];
    pos[0] = TilePos{t0 / A.nrt, t0 % A.nrt};
    expert_state<STAGE, FMT, SH, IDS>(A, S, act, pos[0].a, es[0]);
#pragma unroll
    for (int d = 1; d < D - 1; ++d) {
        pos[d] = d < n ? advance(pos[d - 1], sa, srt, A.nrt) : pos[d - 1];
        if (pos[d].a == es[d - 1].a) es[d] = es[d - 1];
        else expert_state<STAGE, FMT, SH, IDS>(A, S, act, pos[d].a, es[d]);
    }
    u32x4 xr[SPW][4];
    int pidx = 0;
    // the first tile's token operand is requested before any weights, so
    // that resolving its row indices does not wait behind the weight prefetch
    load_tokens<STAGE, SPW, SH, IDS>(A, S, es[0], 0, wv, m, c, xr, pidx, act);
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
        load_tile<FMT, STAGE, SPW, NB, FULL>(A, es[d], pos[d].rt, wv, lane, wr[d], d < n);
    int x_key = es[0].a;
    bool x_raw = true;      // tokens just loaded (not yet in the product type)
    int buf = 0;

    for (int i = 0; i < n; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (i + d < n) {
                const int fd = (d + D - 1) % D, pd = (d + D - 2) % D;
                const bool pf = i + d + D - 1 < n;
                pos[fd] = pf ? advance(pos[pd], sa, srt, A.nrt) : pos[pd];
                dec_step<FMT, STAGE, SPW, KS, NB, YF32, FULL, D, SH, IDS, COH>(
                    A, S, act, red, wr[d], wr[fd], xr, es[d], es[pd], es[fd], pidx, x_key, x_raw, buf,
                    pos[d].rt, pos[fd], pf, lane, wv, m, c);
            }
        }
    }
}

template <int FMT, int STAGE, int SPW, int KS, int NB, bool YF32, bool FULL>
__global__ __launch_bounds__(kWave *KS) void ffn_dec_kernel(DecArgs A) {
    __shared__ float red[2][KS > 1 ? KS - 1 : 1][NB][4][kWave];
    ffn_dec_body<FMT, STAGE, SPW, KS, NB, YF32, FULL, false, false>(A, ShArgs{nullptr, 0},
                                                                    IdsArgs{nullptr, nullptr, 0},
                                                                    red, nullptr);
}

// the same with the shared expert as one more expert of the launch
template <int FMT, int STAGE, int SPW, int KS, int NB, bool YF32, bool FULL>
__global__ __launch_bounds__(kWave *KS) void ffn_dec_kernel_sh(DecArgs A, ShArgs S) {
    __shared__ float red[2][KS > 1 ? KS - 1 : 1][NB][4][kWave];
    ffn_dec_body<FMT, STAGE, SPW, KS, NB, YF32, FULL, true, false>(
        A, S, IdsArgs{nullptr, nullptr, 0}, red, nullptr);
}

// gate/up from the routing ids (the permutation derived in the launch; with
// or without the shared expert). Dynamic LDS: KS x ids_wave_ints(E, n) ints
// (one region per wavefront), then kIdsMaxPairs ints (the workgroup's ids).
template <int FMT, int SPW, int KS, int NB, bool FULL, bool SH>
__global__ __launch_bounds__(kWave *KS) void ffn_dec_kernel_ids(DecArgs A, ShArgs S, IdsArgs I) {
    __shared__ float red[2][KS > 1 ? KS - 1 : 1][NB][4][kWave];
    extern __shared__ __attribute__((aligned(16))) int dec_ids_lds[];
    ffn_dec_body<FMT, 1, SPW, KS, NB, false, FULL, SH, true>(A, S, I, red, dec_ids_lds);
}

// ------------------------------------------------------------- launchers --

// Persistent grid: as many workgroups as can be resident at once.
static int num_cus() {
    static int n = 0;
    if (!n) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
    }
    return n;
}

template <typename K>
static unsigned resident_grid(K kernel, int threads) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
        per_cu <= 0)
        per_cu = 1;
    return (unsigned)(per_cu * num_cus());
}

#ifndef MOE_DEC_WG_PER_CU
#define MOE_DEC_WG_PER_CU 0
#endif
template <int FMT, int STAGE, int SPW, int KS, int NB, bool YF32, bool FULL, bool SH>
static int launch_dec(hipStream_t s, DecArgs A, const ShArgs &S, long slots) {
    static unsigned full = 0;
    if (!full) {
        unsigned res;
        if constexpr (SH)
            res = resident_grid(ffn_dec_kernel_sh<FMT, STAGE, SPW, KS, NB, YF32, FULL>, kWave * KS);
        else
            res = resident_grid(ffn_dec_kernel<FMT, STAGE, SPW, KS, NB, YF32, FULL>, kWave * KS);
        full = MOE_DEC_WG_PER_CU ? MOE_DEC_WG_PER_CU * num_cus() : res;
    }
    // tiles per expert
    A.nrt = STAGE == 1 ? A.I / (8 * NB) : A.H / (16 * NB);
    A.slot_size = num_cus();
    dec_split_weights(STAGE, &A.w_slot, &A.w_pos);
    {   // keep every workgroup's weight at 1/4 or more
        const int last_slot = (int)((full + A.slot_size - 1) / A.slot_size) - 1;
        if (last_slot > 0 && A.w_slot * last_slot + A.w_pos > 0.75f)
            A.w_slot = (0.75f - A.w_pos) / last_slot;
    }
    const long max_tiles = slots * A.nrt;
    const unsigned grid = (unsigned)(max_tiles < (long)full ? max_tiles : (long)full);
    if (grid == 0) return MOE_OK;
    if constexpr (SH)
        MOE_LAUNCH(STAGE == 1 ? K_DEC_GATE_UP : K_DEC_DOWN,
                   (ffn_dec_kernel_sh<FMT, STAGE, SPW, KS, NB, YF32, FULL>), dim3(grid),
                   dim3(kWave * KS), 0, s, A, S);
    else
        MOE_LAUNCH(STAGE == 1 ? K_DEC_GATE_UP : K_DEC_DOWN,
                   (ffn_dec_kernel<FMT, STAGE, SPW, KS, NB, YF32, FULL>), dim3(grid),
                   dim3(kWave * KS), 0, s, A);
    return check_launch();
}

// K split: KS wavefronts x SPW 128-column slabs each. Exact splits for the
// slab counts of the supported shapes; otherwise a bounds-checked split.
// Tiles: stage 1 = 16 gate + 16 up rows (NB = 2); stage 2 = NB2 x 16 rows.
template <int FMT, int STAGE, bool YF32, bool SH>
static int launch_stage(int slabs, hipStream_t s, const DecArgs &A, const ShArgs &S, long slots) {
    // 64-row down tiles, unless that leaves fewer tiles than two workgroups
    // per compute unit (a handful of experts at small batches): then 32
    const bool nb4 = STAGE == 2 && A.H % 64 == 0 && slots * (A.H / 64) >= 2L * num_cus();
#define MOE_ST(SPW_, KS_, FULL_)                                                              \
    return nb4 ? launch_dec<FMT, STAGE, SPW_, KS_, (STAGE == 2 ? 4 : 2), YF32, FULL_, SH>(s, A, S, slots) \
               : launch_dec<FMT, STAGE, SPW_, KS_, 2, YF32, FULL_, SH>(s, A, S, slots)
    switch (slabs) {
        case 1: MOE_ST(1, 1, true);
        case 2: MOE_ST(1, 2, true);
        case 3: MOE_ST(1, 3, true);
        case 4: MOE_ST(1, 4, true);
        case 6: MOE_ST(2, 3, true);
        case 8: MOE_ST(2, 4, true);
        case 12: MOE_ST(3, 4, true);
        case 16:
            // gate/up with fewer tiles than two workgroups per compute unit (a
            // handful of experts): 8 wavefronts per tile shorten each tile
            if (STAGE == 1 && slots * (A.I / 16) < 2L * num_cus()) MOE_ST(2, 8, true);
            MOE_ST(4, 4, true);
        case 24: MOE_ST(3, 8, true);
        case 32: MOE_ST(4, 8, true);
        default: break;
    }
    if (slabs <= 16) MOE_ST(4, 4, false);
    if (slabs <= 32) MOE_ST(4, 8, false);
#undef MOE_ST
    return MOE_EUNSUPPORTED;
}

// Gate/up from the routing ids: launch_dec's grid and split, with the
// permutation's LDS (KS regions) bounding the workgroups per compute unit.
template <int FMT, int SPW, int KS, int NB, bool FULL, bool SH>
static int launch_dec_ids(hipStream_t s, DecArgs A, const ShArgs &S, const IdsArgs &I,
                          long slots) {
    static unsigned full = 0;
    if (!full) {
        const unsigned res = resident_grid(ffn_dec_kernel_ids<FMT, SPW, KS, NB, FULL, SH>,
                                           kWave * KS);
        full = MOE_DEC_WG_PER_CU ? MOE_DEC_WG_PER_CU * num_cus() : res;
    }
    const size_t lds = ((size_t)KS * ids_wave_ints(A.E, I.n) + kIdsMaxPairs) * sizeof(int);
    const size_t red = (size_t)2 * (KS > 1 ? KS - 1 : 1) * NB * 4 * kWave * sizeof(float);
    const unsigned by_lds = (unsigned)(kLdsPerCu / (red + lds)) * (unsigned)num_cus();
    const unsigned fullc = full < by_lds ? full : by_lds;
    A.nrt = A.I / (8 * NB);
    A.slot_size = num_cus();
    dec_split_weights(1, &A.w_slot, &A.w_pos);
    {   // keep every workgroup's weight at 1/4 or more
        const int last_slot = (int)((fullc + A.slot_size - 1) / A.slot_size) - 1;
        if (last_slot > 0 && A.w_slot * last_slot + A.w_pos > 0.75f)
            A.w_slot = (0.75f - A.w_pos) / last_slot;
    }
    const long max_tiles = slots * A.nrt;
    // tile workgroups, plus workgroup 0, which writes the permutation: all
    // resident at once (a tile workgroup that waited for the permutation
    // workgroup's slot would start microseconds late and end the launch late)
    const unsigned tiles_max = fullc > 1 ? fullc - 1 : 1;
    const unsigned grid = (unsigned)(max_tiles < (long)tiles_max ? max_tiles : (long)tiles_max);
    MOE_LAUNCH(K_DEC_GATE_UP, (ffn_dec_kernel_ids<FMT, SPW, KS, NB, FULL, SH>), dim3(grid + 1),
               dim3(kWave * KS), lds, s, A, S, I);
    return check_launch();
}

// Stage 1 shapes as launch_stage.
template <int FMT, bool SH>
static int launch_stage_ids(int slabs, hipStream_t s, const DecArgs &A, const ShArgs &S,
                            const IdsArgs &I, long slots) {
#define MOE_STI(SPW_, KS_, FULL_) return launch_dec_ids<FMT, SPW_, KS_, 2, FULL_, SH>(s, A, S, I, slots)
    switch (slabs) {
        case 1: MOE_STI(1, 1, true);
        case 2: MOE_STI(1, 2, true);
        case 3: MOE_STI(1, 3, true);
        case 4: MOE_STI(1, 4, true);
        case 6: MOE_STI(2, 3, true);
        case 8: MOE_STI(2, 4, true);
        case 12: MOE_STI(3, 4, true);
        case 16:
            if (slots * (A.I / 16) < 2L * num_cus()) MOE_STI(2, 8, true);
            MOE_STI(4, 4, true);
        case 24: MOE_STI(3, 8, true);
        case 32: MOE_STI(4, 8, true);
        default: break;
    }
    if (slabs <= 16) MOE_STI(4, 4, false);
    if (slabs <= 32) MOE_STI(4, 8, false);
#undef MOE_STI
    return MOE_EUNSUPPORTED;
}

// Whether the gate/up launch can derive the permutation from the ids (host
// check, no device work).
static bool ffn_ids_supported(int fmt, int T, int k, int E) {
    const long n = (long)T * k;
    return fmt == MOE_W_MXFP4 && E <= kIdsMaxE && n >= 1 && n <= kIdsMaxPairs;
}

// The permutation (from the ids, in the gate/up launch) and the expert FFN:
// offsets, sorted_pair and pair_row are written as moe_permute writes them.
template <int FMT, bool SH>
static int ffn_decode_ids_fmt(const uint16_t *x, const int32_t *ids, const moe_expert_w *experts,
                              const moe_expert_w *shared, int T, int k, int H, int I, int E,
                              void *y, int y_is_fp32, int32_t *offsets, int32_t *sorted_pair,
                              int32_t *pair_row, uint16_t *act, hipStream_t s) {
    const long n_pairs = (long)T * k;
    const long slots = (n_pairs < E ? n_pairs : E) + n_pairs / kPass +
                       (SH ? (T + kPass - 1) / kPass : 0);
    const ShArgs S{shared, T, T * k};
    const IdsArgs ia{ids, pair_row, (int)n_pairs};
    DecArgs a1{x, sorted_pair, offsets, experts, act, k, H, H, I, E, 0, 1, 0.0f, 0.0f};
    int rc = launch_stage_ids<FMT, SH>((H + 127) / 128, s, a1, S, ia, slots);
    if (rc) return rc;
    DecArgs a2{act, sorted_pair, offsets, experts, y, k, I, H, I, E, 0, 1, 0.0f, 0.0f};
    if (y_is_fp32) return launch_stage<FMT, 2, true, SH>((I + 127) / 128, s, a2, S, slots);
    return launch_stage<FMT, 2, false, SH>((I + 127) / 128, s, a2, S, slots);
}

template <int FMT, bool SH>
static int ffn_decode_fmt(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
                          const moe_expert_w *experts, const moe_expert_w *shared, int T, int k,
                          int H, int I, int E, void *y, int y_is_fp32, uint16_t *act,
                          hipStream_t s) {
    const long n_pairs = (long)T * k;
    // active blocks: at most one per expert with pairs plus one per 16 pairs,
    // and one per 16 tokens of a shared expert
    const long slots = (n_pairs < E ? n_pairs : E) + n_pairs / kPass +
                       (SH ? (T + kPass - 1) / kPass : 0);
    const ShArgs S{shared, T, T * k};
    DecArgs a1{x, sorted_pair, offsets, experts, act, k, H, H, I, E, 0, 1, 0.0f, 0.0f};
    int rc = launch_stage<FMT, 1, false, SH>((H + 127) / 128, s, a1, S, slots);
    if (rc) return rc;
    DecArgs a2{act, sorted_pair, offsets, experts, y, k, I, H, I, E, 0, 1, 0.0f, 0.0f};
    if (y_is_fp32) return launch_stage<FMT, 2, true, SH>((I + 127) / 128, s, a2, S, slots);
    return launch_stage<FMT, 2, false, SH>((I + 127) / 128, s, a2, S, slots);
}

// ---------------------------------------- small batches: down + combine --
//
// At a few tokens the down projection moves a few MB and every launch's
// start-up costs microseconds, so the combine rides in the down launch.
// Workgroup c computes output columns 16c .. 16c+15 for the rows of every
// active expert (the expert's 16-row block c of W2 over K = I), keeps those
// columns of all the layer's rows in LDS, and then writes
//   out[t][16c + i] = bf16( sum_{j<k} w[t][j] y[t*k+j][16c+i]  (+ y_sh[t][16c+i]) ),
// j ascending in fp32 from the bf16 y it also stores: the combine's
// arithmetic on the same y. The activation rows are copied into LDS once per
// workgroup, directly in the matrix-core operand order: 1 KB block
// (g, s, j) holds at byte 16 (m + 16 c) the elements s*128 + 32c + 8j .. +7
// of row 16g + m, so an expert's operand is one 16-byte read per lane and
// MFMA, conflict-free whatever its first row. The four wavefronts take the
// active experts in turn, each with the weights of D experts in registers
// (D - 1 in flight while one is multiplied); two wavefronts per SIMD, so one
// multiplies while the other waits for its weights.
constexpr int kDcMaxT = 16;             // one token pass per expert
// activation rows (T*k routed + T shared): with 16 rows or more (two tokens
// of the 128-expert decode layer, 128 workgroups) the separate down and
// combine launches were as fast or faster in graphs (one workgroup per 16
// output columns then streams several experts' blocks in turn)
constexpr int kDcMaxRows = 15;
constexpr size_t kDcMaxActLds = 128 * 1024;
constexpr int kDcWaves = 8;             // wavefronts per workgroup (two per SIMD)

template <int FMT>
constexpr int wfrag_regs() { return FMT == MOE_W_FP8 ? 8 : 5; }
// experts whose weights are held at once: about 160 registers of weights
template <int FMT, int NS>
constexpr int dc_depth() {
    return 160 / (NS * wfrag_regs<FMT>()) > 4 ? 4 : 160 / (NS * wfrag_regs<FMT>());
}

struct DcArgs {
    const float *topk_w;   // [T][k]
    uint16_t *out;         // [T][H] bf16
    int T, nrows;          // tokens; activation rows (T*k, + T with the shared expert)
};

// An expert of the down + combine launch: rows and W2 resources.
template <int FMT>
struct DcExpert : TensorScale<tensor_scaled(FMT)> {
    int row0, n_e;
    buf_rsrc wr, sr;
};

// Lane q (q < n) of a wavefront describes its q-th expert (active expert
// wv + kDcWaves q): loaded by vector loads once, before the expert loop, and handed
// to the loop by lane reads, so that no expert waits for a load of its
// description (scalar loads there would also hold up the LDS waits).
struct DcMeta {
    int row0, n_e;
    uint64_t w, s;
    float g;
};

__device__ __forceinline__ uint64_t ld_global_u64(const void *p) {
    return *(const MOE_GLOBAL uint64_t *)(p);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
    return (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l) |
           ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l) << 32);
}

// Lane q < n of wavefront wv describes active block wv + kDcWaves q. The
// lookups run with a wavefront-uniform block index (nth is a cross-lane
// search), one per q; the loads then run per lane.
template <int FMT, bool SH>
__device__ __forceinline__ DcMeta dc_meta(const DecArgs &A, const ShArgs &S, const ActiveSet &act,
                                          int wv, int n) {
    DcMeta d{0, 0, 0, 0, 1.0f};
    const int lane = lane_id();
    int e = 0, j = 0;
    for (int q = 0; q < n; ++q) {
        int jq;
        const int eq = act.template nth<SH>(wv + kDcWaves * q, A.E, jq);
        if (lane == q) {
            e = eq;
            j = jq;
        }
    }
    if (lane >= n) return d;
    const bool sh = SH && e == A.E;      // a block of the shared expert's tokens
    d.row0 = (sh ? S.T * A.k : (int)load_u32(A.offsets + e)) + j * kPass;
    d.n_e = min(kPass, (sh ? S.T * (A.k + 1) : (int)load_u32(A.offsets + e + 1)) - d.row0);
    const moe_expert_w *W = sh ? S.shared : A.experts + e;
    d.w = ld_global_u64(&W->w2);
    d.s = ld_global_u64(&W->s2);
    if constexpr (tensor_scaled(FMT)) {
        // the matrix's fp32 scale: after the block scales (NVFP4), or first (FP8)
        const size_t at = FMT == MOE_W_NVFP4 ? (size_t)A.H * A.K / 16 : 0;
        d.g = __uint_as_float(load_u32(reinterpret_cast<const uint8_t *>(d.s) + at));
    }
    return d;
}

template <int FMT>
__device__ __forceinline__ void dc_state(const DecArgs &A, const DcMeta &M, int q,
                                         DcExpert<FMT> &st) {
    st.row0 = __builtin_amdgcn_readlane(M.row0, q);
    st.n_e = __builtin_amdgcn_readlane(M.n_e, q);
    const void *w = reinterpret_cast<const void *>(readlane_u64(M.w, q));
    const void *sc = reinterpret_cast<const void *>(readlane_u64(M.s, q));
    const uint32_t elems = (uint32_t)A.H * (uint32_t)A.K;
    st.wr = make_rsrc(w, FMT == MOE_W_FP8 ? elems : elems / 2);
    st.sr = make_rsrc(sc, FMT == MOE_W_NVFP4 ? elems / 16 : elems / 32);
    if constexpr (tensor_scaled(FMT))
        st.g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(M.g), q));
}

template <int FMT, int NS>
__device__ __forceinline__ void dc_load(const DcExpert<FMT> &st, int rb, int lane,
                                        WFrag<FMT> (&f)[NS], bool on) {
#pragma unroll
    for (int s = 0; s < NS; ++s) f[s].load_block(st.wr, st.sr, (uint32_t)(rb * NS + s), lane, on);
}

// One expert's 16 output columns for its rows (at most 16): the product, the
// bf16 y row pieces to global memory and their values to the LDS rows yl.
template <int FMT, int NS>
__device__ __forceinline__ void dc_expert(const DecArgs &A, const DcExpert<FMT> &st,
                                          WFrag<FMT> (&f)[NS], const uint8_t *actL, float *yl,
                                          const int *spl, int rb, int m, int c, int nrows) {
    int r = st.row0 + m;               // operand row (columns m >= n_e are not used)
    r = r < nrows ? r : nrows - 1;
    const uint8_t *bp = actL + (size_t)(r >> 4) * NS * 4096 + 16 * ((r & 15) + 16 * c);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < NS; ++s) f[s].pin();
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 b = *reinterpret_cast<const u32x4 *>(bp + (s * 4 + j) * 1024);
            if constexpr (f16_path(FMT))
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(f[s].get(j), __builtin_bit_cast(f16x8, b),
                                                            acc, 0, 0, 0);
            else
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f[s].get(j), as_bf16x8(b), acc, 0, 0,
                                                             0);
        }
    if constexpr (tensor_scaled(FMT)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= st.g;
    }
    if (m < st.n_e) {
        const int p = spl[st.row0 + m];
        uint2 pk;
        pk.x = pack_bf16x2(acc[0], acc[1]);
        pk.y = pack_bf16x2(acc[2], acc[3]);
        *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(A.out) + (size_t)p * A.H +
                                   16 * rb + 4 * c) = pk;
        const f32x4 v = {bf16_bits_to_f32(pk.x & 0xFFFFu), bf16_bits_to_f32(pk.x >> 16),
                         bf16_bits_to_f32(pk.y & 0xFFFFu), bf16_bits_to_f32(pk.y >> 16)};
        *reinterpret_cast<f32x4 *>(yl + p * 16 + 4 * c) = v;
    }
}

template <int FMT, int NS, bool SH>
__global__ __launch_bounds__(kWave *kDcWaves) void ffn_dc_kernel(DecArgs A, ShArgs S, DcArgs C) {
    extern __shared__ __attribute__((aligned(16))) uint8_t dc_lds[];
    constexpr int D = dc_depth<FMT, NS>();
    static_assert(D >= 2, "down+combine needs two weight buffers");
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int m = lane & 15, c = lane >> 4;
    const int rb = blockIdx.x;
    const int nrows = C.nrows, ngroups = (nrows + 15) / 16, nk = C.T * A.k;
    uint8_t *actL = dc_lds;
    float *yl = reinterpret_cast<float *>(dc_lds + (size_t)ngroups * NS * 4096);
    int *spl = reinterpret_cast<int *>(yl + nrows * 16);
    float *wl = reinterpret_cast<float *>(spl + nrows);

    ActiveSet act;
    act.template init<SH>(A.offsets, A.E, S);
    // this wavefront's experts: active experts wv, wv + kDcWaves, ...
    const int nmine = act.count > wv ? (act.count - wv + kDcWaves - 1) / kDcWaves : 0;
    const DcMeta meta = dc_meta<FMT, SH>(A, S, act, wv, nmine);
    DcExpert<FMT> es[D];
    WFrag<FMT> wr[D][NS];
    if (nmine > 0) {
#pragma unroll
        for (int d = 0; d < D - 1; ++d) {
            dc_state<FMT>(A, meta, d < nmine ? d : nmine - 1, es[d]);
            dc_load<FMT, NS>(es[d], rb, lane, wr[d], d < nmine);
        }
    }
    // the activation rows into LDS (rows past the end repeat the last one)
    const uint16_t *actg = A.src;
    const int ndma = ngroups * NS * 4;
    for (int d = wv; d < ndma; d += kDcWaves) {
        const int g = d / (NS * 4), s = (d >> 2) % NS, j = d & 3;
        int row = 16 * g + m;
        row = row < nrows ? row : nrows - 1;
        lds_dma16(actg + (size_t)row * A.K + s * 128 + 32 * c + 8 * j, actL + (size_t)d * 1024);
    }
    // each row's pair (the shared expert's rows are their own) and the weights
    const int tid = threadIdx.x;
    if (tid < nrows) spl[tid] = tid < nk ? A.sorted_pair[tid] : tid;
    if (tid < nk) wl[tid] = C.topk_w[tid];
    wait_vm<0>();
    __syncthreads();

    if (nmine > 0) {
        for (int i = 0; i < nmine; i += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                if (i + d < nmine) {
                    // prefetch the expert D - 1 ahead into the buffer freed last
                    const int fd = (d + D - 1) % D, qn = i + d + D - 1;
                    const bool pf = qn < nmine;
                    if (pf) dc_state<FMT>(A, meta, qn, es[fd]);
                    else es[fd] = es[d];
                    dc_load<FMT, NS>(es[fd], rb, lane, wr[fd], pf);
                    dc_expert<FMT, NS>(A, es[d], wr[d], actL, yl, spl, rb, m, c, nrows);
                }
            }
        }
    }
    __syncthreads();
    const int t = tid >> 4, col = tid & 15;
    if (t < C.T) {
        float acc = 0.0f;
        for (int j = 0; j < A.k; ++j) acc += wl[t * A.k + j] * yl[(t * A.k + j) * 16 + col];
        if (SH) acc += yl[(nk + t) * 16 + col];
        C.out[(size_t)t * A.H + 16 * rb + col] = (uint16_t)f32_to_bf16_bits(acc);
    }
}

static size_t dc_lds_bytes(int nrows, int ns, int nk) {
    return (size_t)((nrows + 15) / 16) * ns * 4096 + (size_t)nrows * 16 * 4 + (size_t)nrows * 4 +
           (size_t)nk * 4;
}

template <int FMT, int NS, bool SH>
static int launch_dc(hipStream_t s, const DecArgs &A, const ShArgs &S, const DcArgs &C) {
    const size_t lds = dc_lds_bytes(C.nrows, NS, C.T * A.k);
    static bool attr = false;
    if (!attr) {
        if (int rc = check_hip(hipFuncSetAttribute(
                reinterpret_cast<const void *>(&ffn_dc_kernel<FMT, NS, SH>),
                hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kDcMaxActLds + 8192))))
            return rc;
        attr = true;
    }
    MOE_LAUNCH(K_DEC_DOWN, (ffn_dc_kernel<FMT, NS, SH>), dim3((unsigned)(A.H / 16)),
               dim3(kWave * kDcWaves), lds,
               s, A, S, C);
    return check_launch();
}

// Whether the down + combine launch takes this batch (host check, no device work).
static bool dc_eligible(int fmt, int T, int k, bool sh, int H, int I) {
    if (fmt != MOE_W_MXFP4 && fmt != MOE_W_NVFP4 && fmt != MOE_W_FP8) return false;
    const int nrows = T * k + (sh ? T : 0), ns = I / 128;
    if (T < 1 || T > kDcMaxT || nrows > kDcMaxRows || H % 16 || I % 128) return false;
    if (ns != 2 && ns != 4 && ns != 6 && ns != 8 && ns != 12 && ns != 16) return false;
    if (fmt == MOE_W_FP8 && ns > 8) return false;    // two buffers of 16 slabs exceed the registers
    return (size_t)((nrows + 15) / 16) * ns * 4096 <= kDcMaxActLds;
}

template <int FMT, bool SH>
static int ffn_decode_comb_fmt(const uint16_t *x, const int32_t *sorted_pair,
                               const int32_t *offsets, const moe_expert_w *experts,
                               const moe_expert_w *shared, const float *topk_w, int T, int k,
                               int H, int I, int E, uint16_t *y, uint16_t *out, uint16_t *act,
                               hipStream_t s) {
    const long n_pairs = (long)T * k;
    const long slots = (n_pairs < E ? n_pairs : E) + n_pairs / kPass +
                       (SH ? (T + kPass - 1) / kPass : 0);
    const ShArgs S{shared, T, T * k};
    DecArgs a1{x, sorted_pair, offsets, experts, act, k, H, H, I, E, 0, 1, 0.0f, 0.0f};
    int rc = launch_stage<FMT, 1, false, SH>((H + 127) / 128, s, a1, S, slots);
    if (rc) return rc;
    const DecArgs a2{act, sorted_pair, offsets, experts, y, k, I, H, I, E, 0, 1, 0.0f, 0.0f};
    const DcArgs C{topk_w, out, T, T * k + (SH ? T : 0)};
    switch (I / 128) {
        case 2: return launch_dc<FMT, 2, SH>(s, a2, S, C);
        case 4: return launch_dc<FMT, 4, SH>(s, a2, S, C);
        case 6: return launch_dc<FMT, 6, SH>(s, a2, S, C);
        case 8: return launch_dc<FMT, 8, SH>(s, a2, S, C);
        default: break;
    }
    if constexpr (FMT != MOE_W_FP8) {
        if (I / 128 == 12) return launch_dc<FMT, 12, SH>(s, a2, S, C);
        if (I / 128 == 16) return launch_dc<FMT, 16, SH>(s, a2, S, C);
    }
    return MOE_EUNSUPPORTED;
}

// From the routing ids, with the down projection and the combine in one
// launch (the permutation written by the gate/up launch's workgroup 0, read
// by the down + combine launch); MOE_EUNSUPPORTED (before any device work)
// when the batch does not fit that launch.
template <int FMT, bool SH>
static int ffn_decode_ids_comb_fmt(const uint16_t *x, const int32_t *ids,
                                   const moe_expert_w *experts, const moe_expert_w *shared,
                                   const float *topk_w, int T, int k, int H, int I, int E,
                                   uint16_t *y, uint16_t *out, int32_t *offsets,
                                   int32_t *sorted_pair, int32_t *pair_row, uint16_t *act,
                                   hipStream_t s) {
    if (!dc_eligible(FMT, T, k, SH, H, I)) return MOE_EUNSUPPORTED;
    const long n_pairs = (long)T * k;
    const long slots = (n_pairs < E ? n_pairs : E) + n_pairs / kPass +
                       (SH ? (T + kPass - 1) / kPass : 0);
    const ShArgs S{shared, T, T * k};
    const IdsArgs ia{ids, pair_row, (int)n_pairs};
    DecArgs a1{x, sorted_pair, offsets, experts, act, k, H, H, I, E, 0, 1, 0.0f, 0.0f};
    int rc = launch_stage_ids<FMT, SH>((H + 127) / 128, s, a1, S, ia, slots);
    if (rc) return rc;
    const DecArgs a2{act, sorted_pair, offsets, experts, y, k, I, H, I, E, 0, 1, 0.0f, 0.0f};
    const DcArgs C{topk_w, out, T, T * k + (SH ? T : 0)};
    switch (I / 128) {   // the slab counts dc_eligible admits
        case 2: return launch_dc<FMT, 2, SH>(s, a2, S, C);
        case 4: return launch_dc<FMT, 4, SH>(s, a2, S, C);
        case 6: return launch_dc<FMT, 6, SH>(s, a2, S, C);
        case 8: return launch_dc<FMT, 8, SH>(s, a2, S, C);
        case 12: return launch_dc<FMT, 12, SH>(s, a2, S, C);
        case 16: return launch_dc<FMT, 16, SH>(s, a2, S, C);
        default: return MOE_EUNSUPPORTED;
    }
}

#define MOE_DC_FMT(F, SH)                                                                      \
    return ffn_decode_comb_fmt<F, SH>(x, sorted_pair, offsets, experts, shared, topk_w, T, k, H, \
                                      I, E, y, out, act, s)
#define MOE_DC_DISPATCH(SH)                                                                    \
    if (!dc_eligible(fmt, T, k, SH, H, I)) return MOE_EUNSUPPORTED;                             \
    if (fmt == MOE_W_MXFP4) MOE_DC_FMT(MOE_W_MXFP4, SH);                                       \
    if (fmt == MOE_W_NVFP4) MOE_DC_FMT(MOE_W_NVFP4, SH);                                       \
    MOE_DC_FMT(MOE_W_FP8, SH)

#define MOE_DEC_FMT(F, SH)                                                                     \
    return ffn_decode_fmt<F, SH>(x, sorted_pair, offsets, experts, shared, T, k, H, I, E, y,   \
                                 y_is_fp32, act, s)
#define MOE_DEC_DISPATCH(SH)                                                                   \
    if (fmt == MOE_W_MXFP4) MOE_DEC_FMT(MOE_W_MXFP4, SH);                                      \
    if (fmt == MOE_W_NVFP4) MOE_DEC_FMT(MOE_W_NVFP4, SH);                                      \
    if (fmt == MOE_W_FP8) MOE_DEC_FMT(MOE_W_FP8, SH);                                          \
    MOE_DEC_FMT(MOE_W_BF16, SH)

// The kernels with the shared-expert path are instantiated in a translation
// unit of their own (ffn_decode_shared.hip), so that the two sets compile in
// parallel and the routed-only kernels carry none of that path.
#if defined(MOE_DEC_SMALL_UNIT)
// (the single-launch kernels of ffn_small.hip follow this file there)
#elif !defined(MOE_DEC_SHARED_UNIT)
int ffn_decode_ids_comb(const uint16_t *x, const int32_t *ids, const moe_expert_w *experts,
                        int fmt, const float *topk_w, int T, int k, int H, int I, int E,
                        uint16_t *y, uint16_t *out, int32_t *offsets, int32_t *sorted_pair,
                        int32_t *pair_row, uint16_t *act, hipStream_t s) {
    if (!ffn_ids_supported(fmt, T, k, E)) return MOE_EUNSUPPORTED;
    return ffn_decode_ids_comb_fmt<MOE_W_MXFP4, false>(x, ids, experts, nullptr, topk_w, T, k, H,
                                                       I, E, y, out, offsets, sorted_pair,
                                                       pair_row, act, s);
}
int ffn_decode_ids(const uint16_t *x, const int32_t *ids, const moe_expert_w *experts, int fmt,
                   int T, int k, int H, int I, int E, void *y, int y_is_fp32, int32_t *offsets,
                   int32_t *sorted_pair, int32_t *pair_row, uint16_t *act, hipStream_t s) {
    if (!ffn_ids_supported(fmt, T, k, E)) return MOE_EUNSUPPORTED;
    return ffn_decode_ids_fmt<MOE_W_MXFP4, false>(x, ids, experts, nullptr, T, k, H, I, E, y,
                                                  y_is_fp32, offsets, sorted_pair, pair_row, act,
                                                  s);
}
int ffn_decode(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
               const moe_expert_w *experts, int fmt, int T, int k, int H, int I, int E, void *y,
               int y_is_fp32, uint16_t *act, hipStream_t s) {
    const moe_expert_w *shared = nullptr;
    MOE_DEC_DISPATCH(false);
}
// Gate/up, then down + combine in one launch; MOE_EUNSUPPORTED (before any
// device work) when the batch does not fit that launch.
int ffn_decode_comb(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
                    const moe_expert_w *experts, int fmt, const float *topk_w, int T, int k,
                    int H, int I, int E, uint16_t *y, uint16_t *out, uint16_t *act, hipStream_t s) {
    const moe_expert_w *shared = nullptr;
    MOE_DC_DISPATCH(false);
}
#else
int ffn_decode_ids_comb_shared(const uint16_t *x, const int32_t *ids,
                               const moe_expert_w *experts, const moe_expert_w *shared, int fmt,
                               const float *topk_w, int T, int k, int H, int I, int E,
                               uint16_t *y, uint16_t *out, int32_t *offsets,
                               int32_t *sorted_pair, int32_t *pair_row, uint16_t *act,
                               hipStream_t s) {
    if (!ffn_ids_supported(fmt, T, k, E)) return MOE_EUNSUPPORTED;
    return ffn_decode_ids_comb_fmt<MOE_W_MXFP4, true>(x, ids, experts, shared, topk_w, T, k, H,
                                                      I, E, y, out, offsets, sorted_pair,
                                                      pair_row, act, s);
}
int ffn_decode_ids_shared(const uint16_t *x, const int32_t *ids, const moe_expert_w *experts,
                          const moe_expert_w *shared, int fmt, int T, int k, int H, int I, int E,
                          void *y, int y_is_fp32, int32_t *offsets, int32_t *sorted_pair,
                          int32_t *pair_row, uint16_t *act, hipStream_t s) {
    if (!ffn_ids_supported(fmt, T, k, E)) return MOE_EUNSUPPORTED;
    return ffn_decode_ids_fmt<MOE_W_MXFP4, true>(x, ids, experts, shared, T, k, H, I, E, y,
                                                 y_is_fp32, offsets, sorted_pair, pair_row, act,
                                                 s);
}
int ffn_decode_shared(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
                      const moe_expert_w *experts, const moe_expert_w *shared, int fmt, int T,
                      int k, int H, int I, int E, void *y, int y_is_fp32, uint16_t *act,
                      hipStream_t s) {
    MOE_DEC_DISPATCH(true);
}
int ffn_decode_comb_shared(const uint16_t *x, const int32_t *sorted_pair,
                           const int32_t *offsets, const moe_expert_w *experts,
                           const moe_expert_w *shared, int fmt, const float *topk_w, int T,
                           int k, int H, int I, int E, uint16_t *y, uint16_t *out, uint16_t *act,
                           hipStream_t s) {
    MOE_DC_DISPATCH(true);
}
#endif
#undef MOE_DEC_DISPATCH
#undef MOE_DEC_FMT
#undef MOE_DC_DISPATCH
#undef MOE_DC_FMT

}  // namespace moe
