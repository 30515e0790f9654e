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
// Work decomposition (both stages): a tile is two 16-row blocks of one
// touched expert over the full contraction length K; the KS wavefronts of a
// workgroup split K, and their partial sums meet in LDS (fixed order). Each
// workgroup owns a contiguous range of the U * tiles_per_expert tiles (U =
// experts with pairs, counted on the device), so the grid is fixed and no
// host round trip is needed. While a tile is being multiplied, the next
// tile's weights are already in flight; the token operand stays in registers
// while consecutive tiles belong to the same expert.
//   stage 1: blocks = 16 gate rows and the matching 16 up rows of W13 (K = H);
//            epilogue a = silu(g) * u -> act[sorted row][I] (bf16).
//   stage 2: blocks = 32 consecutive rows of W2 (K = I);
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
// index E after the routed ones. When no routed expert has more than 16 rows,
// its T token rows are cut into blocks of one token pass (16 rows), each one
// more active expert: so the launch keeps its contiguous tile order (one
// expert over T > 16 rows would switch it to the strided order), and the
// blocks read the same weights close together in time (mostly from cache).
// When some routed expert needs several passes anyway, it stays one expert
// over all T rows. Token t's activation and output row is base + t, base =
// T*k. A second kernel argument, so that launches without it keep the
// argument layout (and scalar registers) they had.
struct ShArgs {
    const moe_expert_w *shared;
    int T, base;
};

// Experts that received at least one pair, as a bitmask (E <= 512), computed
// by the whole wavefront from one round of loads; lookups afterwards are
// scalar. With a shared expert it is one more active expert, the last, with
// expert index E and all T tokens as its rows.
struct ActiveSet {
    uint64_t w[8];
    int count;               // active experts, the shared one included
    int routed;              // active routed experts
    const moe_expert_w *sh_w;  // shared expert's weights and tokens (SH launches)
    int sh_T;
    bool multi_pass;         // some routed expert has more rows than one token pass
    template <bool SH>
    __device__ __forceinline__ void init(const int32_t *__restrict__ offsets, int E,
                                         const ShArgs &S) {
        count = 0;
        int cnt[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = i * kWave + lane_id();
            cnt[i] = e < E ? offsets[e + 1] - offsets[e] : 0;
        }
        uint64_t many = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            w[i] = __ballot(cnt[i] > 0);
            many |= __ballot(cnt[i] > kPass);
            count += __popcll(w[i]);
        }
        routed = count;
        multi_pass = many != 0;
        // the shared expert: blocks of 16 tokens, or one block over all T when
        // the launch has several passes anyway (shared_block)
        if constexpr (SH) {
            count += multi_pass ? 1 : (S.T + kPass - 1) / kPass;
            sh_w = S.shared;
            sh_T = S.T;
        }
    }
    // index of the a-th (0-based) active expert; a < count
    // (a shared-expert block: E)
    template <bool SH>
    __device__ __forceinline__ int nth(int a, int E) const {
        if constexpr (SH) {
            if (a >= routed) return E;
        }
        int base = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = __popcll(w[i]);
            if (a < c) {
                uint64_t m = w[i];
                for (int r = 0; r < a; ++r) m &= m - 1;
                return i * kWave + __ffsll((long long)m) - 1;
            }
            a -= c;
            base += c;
        }
        return -1;
    }
};

struct DecArgs {
    const uint16_t *src;            // B-operand rows: x [T][H] (stage 1) or act [T*k][I] (stage 2)
    const int32_t *sorted_pair;
    const int32_t *offsets;
    const moe_expert_w *experts;
    void *out;                      // act (stage 1) or y (stage 2)
    int k, K, H, I, E, nrt;         // nrt: tiles per expert
};


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
template <int STAGE, int FMT, bool SH>
__device__ __forceinline__ void expert_state(const DecArgs &A, const ShArgs &S,
                                             const ActiveSet &act, int a, ExpertState<FMT> &st) {
    st.a = a;
    st.e = act.template nth<SH>(a, A.E);
    const MOE_CONST int32_t *off = as_scalar(A.offsets);
    const bool sh = SH && st.e == A.E;        // a block of the shared expert's tokens
    const int bs = act.multi_pass ? act.sh_T : kPass;   // (its rows per block)
    const int j = a - act.routed;             // (which block)
    st.row0 = sh ? act.sh_T * A.k + j * bs : off[st.e];
    st.n_e = sh ? min(bs, act.sh_T - j * bs) : off[st.e + 1] - st.row0;
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
template <int STAGE, int SPW, bool SH, class ES>
__device__ __forceinline__ void load_tokens(const DecArgs &A, const ShArgs &S, const ES &st,
                                            int p, int wv, int m, int c, u32x4 (&xr)[SPW][4],
                                            int &pidx) {
    const int nblk = A.K / 32;
    const int r = p * kPass + m;
    const bool has = r < st.n_e;
    const uint16_t *row;
    // shared-expert block: row r is token row0 - base + r; its output row is row0 + r
    const bool sh = SH && st.e == A.E;
    if (STAGE == 1) {
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
template <int FMT, int STAGE, int SPW, int KS, int NB, bool YF32, bool FULL, int D, bool SH>
__device__ __forceinline__ void dec_step(const DecArgs &A, const ShArgs &S, const ActiveSet &act,
                                         float (&red)[2][KS > 1 ? KS - 1 : 1][NB][4][kWave],
                                         WFrag<FMT> (&wc)[SPW][NB], WFrag<FMT> (&wn)[SPW][NB],
                                         u32x4 (&xr)[SPW][4], const ExpertState<FMT> &cur,
                                         const ExpertState<FMT> &prev, ExpertState<FMT> &nxt,
                                         int &pidx, int &x_key, bool &x_raw, int &buf, int rt,
                                         TilePos pn, bool pf, int lane, int wv, int m, int c) {

        // token operand for the first pass of this tile (loaded before the next
        // prefetch, so that waiting for it does not wait for the prefetched weights)
        if (x_key != cur.a * 4096) {
            load_tokens<STAGE, SPW, SH>(A, S, cur, 0, wv, m, c, xr, pidx);
            x_key = cur.a * 4096;
            x_raw = true;
        }
        // prefetch the tile D - 1 steps ahead (position pn, present if pf);
        // `prev` holds the state of the tile before it. Issued, switched off,
        // also past the end (see buf_rsrc).
        const int an = pf ? pn.a : prev.a;
        if (an != prev.a) expert_state<STAGE, FMT, SH>(A, S, act, an, nxt);
        else nxt = prev;
        load_tile<FMT, STAGE, SPW, NB, FULL>(A, nxt, pf ? pn.rt : 0, wv, lane, wn, pf);
        for (int p = 0; p * kPass < cur.n_e; ++p) {
            if (p > 0) {   // more than 16 tokens: next 16 of this expert
                load_tokens<STAGE, SPW, SH>(A, S, cur, p, wv, m, c, xr, pidx);
                x_key = cur.a * 4096 + p;
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
                            *reinterpret_cast<uint2 *>(actp + (rt * H2 + b) * 16 + 4 * c) = pk;
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

template <int FMT, int STAGE, int SPW, int KS, int NB, bool YF32, bool FULL, bool SH>
__device__ __forceinline__ void ffn_dec_body(const DecArgs &A, const ShArgs &S,
                                             float (&red)[2][KS > 1 ? KS - 1 : 1][NB][4][kWave]) {
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wavefront-uniform
    const int m = lane & 15, c = lane >> 4;

    ActiveSet act;
    act.template init<SH>(A.offsets, A.E, S);
    // Tiles are active-expert-major. Workgroups take contiguous ranges, which
    // keep an expert's token operand in registers across its tiles, unless some
    // expert has more rows than one token pass: then workgroup b takes tiles b,
    // b + g, b + 2g, .. (g workgroups), so the tiles of the few experts with
    // many rows (skewed popularity) spread over many workgroups instead of
    // stretching the ones that hold them.
    const int total = act.count * A.nrt;
    int t0, n, ts;
    if (act.multi_pass) {
        t0 = blockIdx.x;
        ts = gridDim.x;
        n = t0 < total ? (total - t0 + ts - 1) / ts : 0;
    } else {
        t0 = (int)((long)blockIdx.x * total / gridDim.x);
        n = (int)(((long)blockIdx.x + 1) * total / gridDim.x) - t0;
        ts = 1;
    }
    if (n <= 0) return;
    const int sa = ts / A.nrt, srt = ts % A.nrt;

    // D register buffers used in turn: tile i computes from one while the
    // weights of tiles i+1 .. i+D-1 are in flight into the others (no copies
    // between them, so nothing waits for a prefetch before it is needed).
    // Slots past the end repeat the last tile's position and load nothing.
    constexpr int D = STAGE == 2 ? kDepth2 : kDepth;
    ExpertState<FMT> es[D];
    TilePos pos[D];
    WFrag<FMT> wr[D][SPW][NB];
    pos[0] = TilePos{t0 / A.nrt, t0 % A.nrt};
    expert_state<STAGE, FMT, SH>(A, S, act, pos[0].a, es[0]);
#pragma unroll
    for (int d = 1; d < D - 1; ++d) {
        pos[d] = d < n ? advance(pos[d - 1], sa, srt, A.nrt) : pos[d - 1];
        if (pos[d].a == es[d - 1].a) es[d] = es[d - 1];
        else expert_state<STAGE, FMT, SH>(A, S, act, pos[d].a, es[d]);
    }
    // the first tile's token operand is requested before any weights, so that
    // resolving its row indices does not wait behind the weight prefetch
    u32x4 xr[SPW][4];
    int pidx = 0;
    load_tokens<STAGE, SPW, SH>(A, S, es[0], 0, wv, m, c, xr, pidx);
    int x_key = es[0].a * 4096;
    bool x_raw = true;      // tokens just loaded (not yet in the product type)
    int buf = 0;
#pragma unroll
    for (int d = 0; d < D - 1; ++d)
        load_tile<FMT, STAGE, SPW, NB, FULL>(A, es[d], pos[d].rt, wv, lane, wr[d], d < n);

    for (int i = 0; i < n; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (i + d < n) {
                const int fd = (d + D - 1) % D, pd = (d + D - 2) % D;
                const bool pf = i + d + D - 1 < n;
                pos[fd] = pf ? advance(pos[pd], sa, srt, A.nrt) : pos[pd];
                dec_step<FMT, STAGE, SPW, KS, NB, YF32, FULL, D, SH>(
                    A, S, act, red, wr[d], wr[fd], xr, es[d], es[pd], es[fd], pidx, x_key, x_raw, buf,
                    pos[d].rt, pos[fd], pf, lane, wv, m, c);
            }
        }
    }
}

template <int FMT, int STAGE, int SPW, int KS, int NB, bool YF32, bool FULL>
__global__ __launch_bounds__(kWave *KS) void ffn_dec_kernel(DecArgs A) {
    __shared__ float red[2][KS > 1 ? KS - 1 : 1][NB][4][kWave];
    ffn_dec_body<FMT, STAGE, SPW, KS, NB, YF32, FULL, false>(A, ShArgs{nullptr, 0}, red);
}

// the same with the shared expert as one more expert of the launch
template <int FMT, int STAGE, int SPW, int KS, int NB, bool YF32, bool FULL>
__global__ __launch_bounds__(kWave *KS) void ffn_dec_kernel_sh(DecArgs A, ShArgs S) {
    __shared__ float red[2][KS > 1 ? KS - 1 : 1][NB][4][kWave];
    ffn_dec_body<FMT, STAGE, SPW, KS, NB, YF32, FULL, true>(A, S, red);
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

template <int FMT, bool SH>
static int ffn_decode_fmt(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
                          const moe_expert_w *experts, const moe_expert_w *shared, int T, int k,
                          int H, int I, int E, void *y, int y_is_fp32, uint16_t *act,
                          hipStream_t s) {
    const long n_pairs = (long)T * k;
    // a shared expert adds one active expert per 16 tokens
    const long slots = (n_pairs < E ? n_pairs : E) + (SH ? (T + kPass - 1) / kPass : 0);
    const ShArgs S{shared, T, T * k};
    DecArgs a1{x, sorted_pair, offsets, experts, act, k, H, H, I, E, 0};
    int rc = launch_stage<FMT, 1, false, SH>((H + 127) / 128, s, a1, S, slots);
    if (rc) return rc;
    DecArgs a2{act, sorted_pair, offsets, experts, y, k, I, H, I, E, 0};
    if (y_is_fp32) return launch_stage<FMT, 2, true, SH>((I + 127) / 128, s, a2, S, slots);
    return launch_stage<FMT, 2, false, SH>((I + 127) / 128, s, a2, S, slots);
}

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
#ifndef MOE_DEC_SHARED_UNIT
int ffn_decode(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
               const moe_expert_w *experts, int fmt, int T, int k, int H, int I, int E, void *y,
               int y_is_fp32, uint16_t *act, hipStream_t s) {
    const moe_expert_w *shared = nullptr;
    MOE_DEC_DISPATCH(false);
}
#else
int ffn_decode_shared(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
                      const moe_expert_w *experts, const moe_expert_w *shared, int fmt, int T,
                      int k, int H, int I, int E, void *y, int y_is_fp32, uint16_t *act,
                      hipStream_t s) {
    MOE_DEC_DISPATCH(true);
}
#endif
#undef MOE_DEC_DISPATCH
#undef MOE_DEC_FMT

}  // namespace moe
