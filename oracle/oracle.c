/*
 * CPU oracle for the routed MoE expert layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this file's library. The GPU library never links, includes or calls it,
 * and it shares no source with the GPU library.
 *
 * What it computes is the plain definition of the layer the FreeToken pages
 * describe: each token is sent to a few routed experts (winzheng.com page,
 * "Why Now": six routed experts per token per decoder layer, the rest of the
 * FP4-quantised pool idle), each expert being a SwiGLU feed-forward block whose
 * weights are stored in MXFP4, NVFP4, FP8 or BF16 (aimodeling.com/en page,
 * "Reported Numbers and Ecosystem Position", lists these formats).
 * The pages do not spell out the routing function, the FFN form or the
 * combine; the readings taken are:
 *   - routing selects the k largest logits (ties: lower expert index first) and
 *     weights them by a softmax renormalised over the selected k;
 *   - expert FFN: y = W2 (silu(W1 x) * (W3 x)), W1/W3 stacked as W13;
 *   - combine: out[t] = sum_j w[t][j] * y[t,j] (+ shared expert, weight 1).
 *
 * Arithmetic: weights decoded exactly, accumulation in double, no blocking or
 * reordering beyond what the definition states, single thread, no intrinsics.
 * The one place where fp32 is used on purpose is the router gate: the gate
 * logits decide an integer (the expert choice), so they are formed in fp32 in
 * the same fixed summation order as the GPU kernel (a 64-lane split by 8-element
 * chunks, then a halving butterfly), which makes the choice reproducible.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- codecs -- */

/* bf16 bits -> double (exact: bf16 is the top half of an IEEE binary32). */
double orc_bf16_to_f64(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* double -> bf16 bits, round to nearest, ties to even, in a single rounding
 * step from the double value. NaN -> canonical quiet NaN. */
uint16_t orc_f64_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    uint16_t sign = (uint16_t)(neg << 15);
    if (a == 0.0) return sign;
    /* largest finite bf16: (2 - 2^-7) * 2^127; halfway to the next binade
     * rounds up to infinity */
    const double max_bf16 = ldexp(255.0 / 128.0, 127);
    const double overflow_mid = ldexp(511.0 / 256.0, 127);
    if (a >= overflow_mid) return (uint16_t)(sign | 0x7F80);
    if (a > max_bf16) return (uint16_t)(sign | 0x7F7F);
    int e;
    frexp(a, &e);              /* a = m * 2^e, m in [0.5, 1) */
    int exp_unb = e - 1;       /* a = 1.f * 2^exp_unb */
    if (exp_unb < -126) exp_unb = -126;      /* subnormal range: fixed quantum */
    /* quantum of an 8-bit significand (7 stored bits) in this binade */
    double q = ldexp(1.0, exp_unb - 7);
    double n = a / q;          /* exact: power-of-two scaling */
    double fl = floor(n);
    double frac = n - fl;
    double r;
    if (frac > 0.5) r = fl + 1.0;
    else if (frac < 0.5) r = fl;
    else r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double res = r * q;        /* representable */
    float f = (float)res;      /* exact */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

/* E2M1 element (OCP Microscaling v1.0): 1 sign, 2 exponent (bias 1), 1 mantissa.
 * exponent field 0 is subnormal: 0.5 * m. */
double orc_e2m1(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* E8M0 scale: 2^(S-127); 255 encodes NaN. */
double orc_e8m0(int s) {
    if (s == 255) return NAN;
    return ldexp(1.0, s - 127);
}

/* Decode rows [R][K] of MXFP4 (codes [R][K/2], even element in the low
 * nibble; one E8M0 scale per 32 consecutive elements of a row). */
void orc_mxfp4_decode(const uint8_t *codes, const uint8_t *scales, long R, long K, double *out) {
    /* the 16 element values and 256 scale values, tabulated once per call */
    double elem[16], scale[256];
    for (int i = 0; i < 16; ++i) elem[i] = orc_e2m1(i);
    for (int i = 0; i < 256; ++i) scale[i] = orc_e8m0(i);
    for (long r = 0; r < R; ++r)
        for (long c = 0; c < K; ++c) {
            uint8_t byte = codes[r * (K / 2) + c / 2];
            int code = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
            out[r * K + c] = elem[code] * scale[scales[r * (K / 32) + c / 32]];
        }
}

/* E4M3 (OCP 8-bit floating point, the variant without infinities): 1 sign,
 * 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is subnormal
 * (m/8 * 2^-6); S.1111.111 is NaN, so the largest finite value is 448. */
double orc_e4m3(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Decode rows [R][K] of NVFP4 (aimodeling.com/en page, "Reported Numbers and
 * Ecosystem Position", lists NVFP4 among the weight formats): E2M1 codes
 * [R][K/2] (even element in the low nibble), one E4M3 scale per 16
 * consecutive elements of a row (scales [R][K/16]), and one fp32 scale g for
 * the matrix: value = e2m1 * e4m3(scale) * g. */
void orc_nvfp4_decode(const uint8_t *codes, const uint8_t *scales, float g, long R, long K,
                      double *out) {
    for (long r = 0; r < R; ++r)
        for (long c = 0; c < K; ++c) {
            uint8_t byte = codes[r * (K / 2) + c / 2];
            int code = (c % 2 == 0) ? (byte & 15) : (byte >> 4);
            out[r * K + c] = orc_e2m1(code) * orc_e4m3(scales[r * (K / 16) + c / 16]) * (double)g;
        }
}

/* Decode rows [R][K] of FP8 weights: E4M3 codes [R][K] times the matrix's
 * fp32 scale g. */
void orc_fp8_decode(const uint8_t *codes, float g, long R, long K, double *out) {
    for (long i = 0; i < R * K; ++i) out[i] = orc_e4m3(codes[i]) * (double)g;
}

static float read_f32(const uint8_t *p) {
    float f;
    memcpy(&f, p, 4);
    return f;
}

static void decode_bf16_rows(const uint16_t *w, long n, double *out) {
    for (long i = 0; i < n; ++i) out[i] = orc_bf16_to_f64(w[i]);
}

/* ------------------------------------------------------------- router ---- */

/* Gate logits in fp32 in the fixed order described in the file header:
 * lane l (0..63) sums, in ascending h and starting from +0, the products whose
 * 8-element chunk index h/8 is congruent to l mod 64; lanes are then combined
 * by a butterfly with partner distances 32,16,8,4,2,1 (each partial sum adds
 * the partner's partial). Products of two bf16 are exact in fp32. */
void orc_gate_logits_f32(const uint16_t *x, const uint16_t *wg, int T, int H, int E, float *logits) {
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            float lane[64];
            for (int l = 0; l < 64; ++l) lane[l] = 0.0f;
            for (int h = 0; h < H; ++h) {
                float p = (float)orc_bf16_to_f64(x[(long)t * H + h]) *
                          (float)orc_bf16_to_f64(wg[(long)e * H + h]);
                lane[(h / 8) % 64] += p;
            }
            for (int d = 32; d >= 1; d /= 2) {
                float nxt[64];
                for (int l = 0; l < 64; ++l) nxt[l] = lane[l] + lane[l ^ d];
                memcpy(lane, nxt, sizeof(lane));
            }
            logits[(long)t * E + e] = lane[0];
        }
}

/* Same dot products in double (for diagnosing near-ties only). */
void orc_gate_logits_f64(const uint16_t *x, const uint16_t *wg, int T, int H, int E, double *logits) {
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int h = 0; h < H; ++h)
                s += orc_bf16_to_f64(x[(long)t * H + h]) * orc_bf16_to_f64(wg[(long)e * H + h]);
            logits[(long)t * E + e] = s;
        }
}

/* expert a ranks before expert b: larger logit, then lower index */
static int ranks_before(const float *l, int a, int b) {
    if (l[a] > l[b]) return 1;
    if (l[a] < l[b]) return 0;
    return a < b;
}

/* Top-k routing. Per token, the experts are ordered by (logit desc, index asc)
 * with a plain insertion sort and the first k kept, in that order.
 * renormalize=1: w_j = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0)
 *                (= softmax over all E, then renormalised over the k kept)
 * renormalize=0: w_j = exp(l_j - l_max) / sum_{e<E} exp(l_e - l_max)
 * Weights are computed in double; w64 (optional) receives them unrounded.
 * Returns -1 if a logit is not finite, else 0. */
int orc_topk(const float *logits, int T, int E, int k, int renormalize,
             int32_t *ids, float *w, double *w64) {
    int *order = (int *)malloc(sizeof(int) * (size_t)E);
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (long)t * E;
        for (int e = 0; e < E; ++e) {
            if (!isfinite(l[e])) { free(order); return -1; }
            order[e] = e;
        }
        for (int i = 1; i < E; ++i) {
            int cur = order[i], j = i - 1;
            while (j >= 0 && ranks_before(l, cur, order[j])) {
                order[j + 1] = order[j];
                --j;
            }
            order[j + 1] = cur;
        }
        double lmax = (double)l[order[0]];
        double denom = 0.0;
        if (renormalize) {
            for (int j = 0; j < k; ++j) denom += exp((double)l[order[j]] - lmax);
        } else {
            for (int e = 0; e < E; ++e) denom += exp((double)l[e] - lmax);
        }
        for (int j = 0; j < k; ++j) {
            double wj = exp((double)l[order[j]] - lmax) / denom;
            ids[(long)t * k + j] = order[j];
            w[(long)t * k + j] = (float)wj;
            if (w64) w64[(long)t * k + j] = wj;
        }
    }
    free(order);
    return 0;
}

/* ------------------------------------------------------------ permute ---- */

/* Stable counting sort of the T*k (token, slot) pairs p = t*k + j by expert:
 * offsets[e] = number of pairs routed to experts < e (offsets[E] = T*k);
 * sorted_pair[offsets[e] + r] = the r-th pair, in ascending p, routed to e;
 * pair_row[p] = the row of sorted order that holds pair p. */
int orc_permute(const int32_t *ids, int T, int k, int E,
                int32_t *offsets, int32_t *sorted_pair, int32_t *pair_row) {
    long n = (long)T * k;
    int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
    for (int e = 0; e <= E; ++e) offsets[e] = 0;
    for (long p = 0; p < n; ++p) {
        if (ids[p] < 0 || ids[p] >= E) { free(fill); return -1; }
        offsets[ids[p] + 1] += 1;
    }
    for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    for (long p = 0; p < n; ++p) {
        int e = ids[p];
        int32_t row = offsets[e] + fill[e]++;
        sorted_pair[row] = (int32_t)p;
        pair_row[p] = row;
    }
    free(fill);
    return 0;
}

/* ---------------------------------------------------------------- FFN ---- */

/* Host-side view of one expert blob: W13 [2I][H] (rows 0..I-1 gate, I..2I-1
 * up) and W2 [H][I], each bf16 (scales unused), MXFP4 codes + E8M0 scales,
 * NVFP4 codes + E4M3 scales followed by the matrix's fp32 scale, or FP8
 * codes with the scale pointer at the matrix's fp32 scale. */
typedef struct {
    const void *w13;
    const uint8_t *s13;
    const void *w2;
    const uint8_t *s2;
} orc_expert;

static void decode_expert(const orc_expert *x, int fmt, int H, int I, double *w13, double *w2) {
    if (fmt == 0) {
        decode_bf16_rows((const uint16_t *)x->w13, (long)2 * I * H, w13);
        decode_bf16_rows((const uint16_t *)x->w2, (long)H * I, w2);
    } else if (fmt == 1) {
        orc_mxfp4_decode((const uint8_t *)x->w13, x->s13, 2L * I, H, w13);
        orc_mxfp4_decode((const uint8_t *)x->w2, x->s2, H, I, w2);
    } else if (fmt == 2) {
        orc_nvfp4_decode((const uint8_t *)x->w13, x->s13, read_f32(x->s13 + 2L * I * H / 16),
                         2L * I, H, w13);
        orc_nvfp4_decode((const uint8_t *)x->w2, x->s2, read_f32(x->s2 + (long)H * I / 16), H, I,
                         w2);
    } else {
        orc_fp8_decode((const uint8_t *)x->w13, read_f32(x->s13), 2L * I, H, w13);
        orc_fp8_decode((const uint8_t *)x->w2, read_f32(x->s2), H, I, w2);
    }
}

/* SwiGLU expert FFN on a list of rows: row r applies expert row_expert[r] to
 * token row_token[r] of x [T][H] (bf16):
 *   g_i = sum_h x_h W13[i][h],  u_i = sum_h x_h W13[I+i][h]
 *   a_i = g_i / (1 + exp(-g_i)) * u_i
 *   y_n = sum_i a_i W2[n][i]
 * Everything in double. y: [nrows][H]; act (optional): [nrows][I].
 * Each expert is decoded once, then all of its rows are evaluated.
 * fmt: 0 = bf16, 1 = MXFP4, 2 = NVFP4, 3 = FP8. Returns -1 on a bad expert
 * index or allocation. */
int orc_ffn_rows(const uint16_t *x, int H, int I, int fmt, const orc_expert *experts, int E,
                 long nrows, const int32_t *row_token, const int32_t *row_expert,
                 double *y, double *act) {
    double *w13 = (double *)malloc(sizeof(double) * (size_t)2 * I * H);
    double *w2 = (double *)malloc(sizeof(double) * (size_t)H * I);
    double *xr = (double *)malloc(sizeof(double) * (size_t)H);
    double *a = (double *)malloc(sizeof(double) * (size_t)I);
    if (!w13 || !w2 || !xr || !a) { free(w13); free(w2); free(xr); free(a); return -1; }
    for (long r = 0; r < nrows; ++r)
        if (row_expert[r] < 0 || row_expert[r] >= E) { free(w13); free(w2); free(xr); free(a); return -1; }
    for (int e = 0; e < E; ++e) {
        int used = 0;
        for (long r = 0; r < nrows && !used; ++r) used = (row_expert[r] == e);
        if (!used) continue;
        decode_expert(&experts[e], fmt, H, I, w13, w2);
        for (long r = 0; r < nrows; ++r) {
            if (row_expert[r] != e) continue;
            const uint16_t *xt = x + (long)row_token[r] * H;
            for (int h = 0; h < H; ++h) xr[h] = orc_bf16_to_f64(xt[h]);
            for (int i = 0; i < I; ++i) {
                double g = 0.0, u = 0.0;
                const double *wg = w13 + (long)i * H, *wu = w13 + (long)(I + i) * H;
                for (int h = 0; h < H; ++h) {
                    g += xr[h] * wg[h];
                    u += xr[h] * wu[h];
                }
                a[i] = g / (1.0 + exp(-g)) * u;
                if (act) act[r * I + i] = a[i];
            }
            for (int n = 0; n < H; ++n) {
                double s = 0.0;
                const double *w2n = w2 + (long)n * I;
                for (int i = 0; i < I; ++i) s += a[i] * w2n[i];
                y[r * H + n] = s;
            }
        }
    }
    free(w13); free(w2); free(xr); free(a);
    return 0;
}

/* ------------------------------------------------------------ combine ---- */

/* out[t][n] = sum_{j<k} w[t][j] * y[t*k+j][n]  (+ y_shared[t][n], weight 1),
 * in double, j ascending; out_f64 keeps the exact sum, out_bf16 its rounding. */
void orc_combine(const double *y, const float *w, const double *y_shared,
                 long T, int k, int H, double *out_f64, uint16_t *out_bf16) {
    for (long t = 0; t < T; ++t)
        for (int n = 0; n < H; ++n) {
            double s = 0.0;
            for (int j = 0; j < k; ++j) s += (double)w[t * k + j] * y[(t * k + j) * H + n];
            if (y_shared) s += y_shared[t * H + n];
            if (out_f64) out_f64[t * H + n] = s;
            if (out_bf16) out_bf16[t * H + n] = orc_f64_to_bf16(s);
        }
}

/* ------------------------------------------------------- whole layer ---- */

/* The layer for all T tokens: route (from given logits, or from the gate when
 * logits_in is NULL), permute, expert FFN for every routed pair, shared expert
 * (if given), combine. Outputs are optional except out_f64.
 * Returns 0, or -1 on invalid input. */
int orc_moe_layer(const uint16_t *x, const uint16_t *wg, const float *logits_in,
                  int T, int H, int E, int k, int I, int fmt, int renormalize,
                  const orc_expert *experts, const orc_expert *shared,
                  float *logits_out, int32_t *ids, float *w, int32_t *offsets,
                  int32_t *sorted_pair, int32_t *pair_row, double *y_pairs,
                  double *out_f64, uint16_t *out_bf16) {
    long n = (long)T * k;
    int rc = 0;
    float *lg = (float *)malloc(sizeof(float) * (size_t)T * E);
    int32_t *ids_ = ids ? ids : (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    float *w_ = w ? w : (float *)malloc(sizeof(float) * (size_t)n);
    int32_t *off_ = offsets ? offsets : (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *sp_ = sorted_pair ? sorted_pair : (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    int32_t *pr_ = pair_row ? pair_row : (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    double *y_ = y_pairs ? y_pairs : (double *)malloc(sizeof(double) * (size_t)n * H);
    int32_t *tok = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    double *ysh = shared ? (double *)malloc(sizeof(double) * (size_t)T * H) : NULL;
    int32_t *zero = shared ? (int32_t *)calloc((size_t)T, sizeof(int32_t)) : NULL;
    int32_t *seq = shared ? (int32_t *)malloc(sizeof(int32_t) * (size_t)T) : NULL;

    if (logits_in) memcpy(lg, logits_in, sizeof(float) * (size_t)T * E);
    else orc_gate_logits_f32(x, wg, T, H, E, lg);
    if (logits_out) memcpy(logits_out, lg, sizeof(float) * (size_t)T * E);
    if (orc_topk(lg, T, E, k, renormalize, ids_, w_, NULL) != 0) { rc = -1; goto done; }
    if (orc_permute(ids_, T, k, E, off_, sp_, pr_) != 0) { rc = -1; goto done; }
    /* rows in pair order p = t*k + j (the FFN of a pair does not depend on
     * its position in sorted order) */
    for (long p = 0; p < n; ++p) tok[p] = (int32_t)(p / k);
    if (orc_ffn_rows(x, H, I, fmt, experts, E, n, tok, ids_, y_, NULL) != 0) { rc = -1; goto done; }
    if (shared) {
        for (int t = 0; t < T; ++t) seq[t] = t;
        if (orc_ffn_rows(x, H, I, fmt, shared, 1, T, seq, zero, ysh, NULL) != 0) { rc = -1; goto done; }
    }
    orc_combine(y_, w_, ysh, T, k, H, out_f64, out_bf16);
done:
    free(lg);
    if (!ids) free(ids_);
    if (!w) free(w_);
    if (!offsets) free(off_);
    if (!sorted_pair) free(sp_);
    if (!pair_row) free(pr_);
    if (!y_pairs) free(y_);
    free(tok); free(ysh); free(zero); free(seq);
    return rc;
}
