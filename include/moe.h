/*
 * moe.h -- C ABI of the routed MoE expert layer for MI355X (gfx950).
 *
 * The layer is the expert block of a sparse mixture-of-experts decoder: every
 * token is sent to k routed experts out of E, each expert is a SwiGLU
 * feed-forward block with block-scaled FP4 weights, and the k expert outputs
 * are mixed by the router's weights. The FreeToken pages describe this
 * sparsity as what makes edge serving of very large models possible
 * (winzheng.com page, "Why Now of All Times": per token, each of the 43
 * decoder layers uses six routed experts, and since the FP4-quantised pool is
 * far larger than device memory, most experts stay on the host and are copied
 * in when routed to) and list MXFP4, NVFP4, FP8 and BF16
 * weights (aimodeling.com/en page, "Reported Numbers and Ecosystem Position").
 * The expert cache calls follow the pages' global LRU expert cache and
 * full-layer double-buffered prefill streaming (winzheng.com page,
 * "FreeToken's Three-Layer Mechanism"; aimodeling.com/en page, "Three
 * Engineering Cores").
 *
 * Conventions for every call below
 *   - Pointers are device pointers unless marked (host).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream); the call returns once the work is enqueued.
 *   - Return value: MOE_OK (0) or a negative moe_err. Argument errors are
 *     detected before anything is enqueued and leave every output untouched.
 *     A HIP launch/copy failure returns MOE_EHIP; moe_last_hip_error() gives
 *     the HIP code. Faults inside kernels surface at the caller's next
 *     synchronisation, as for any HIP kernel.
 *   - The caller owns and allocates all buffers (activations, logits, ids,
 *     offsets, outputs, workspaces, the expert-cache pool). The layer calls
 *     allocate nothing; only expert_cache_reserve allocates (its small device
 *     table and host metadata).
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - Token-pair numbering: pair p = t*k + j is the j-th expert (in routing
 *     order) of token t.
 *
 * Expert weights (one contiguous blob per expert, described by moe_expert_w):
 * W13 has 2I rows of length H (rows 0..I-1 are the gate projection W1, rows
 * I..2I-1 the up projection W3); W2 has H rows of length I.
 *   Interchange MXFP4 layout (row-major; what moe_pack_mxfp4 reads): rows of
 *     E2M1 codes, two per byte, the even element in the low nibble; one E8M0
 *     scale byte per 32 consecutive elements of a row (scales [rows][K/32]).
 *   Kernel MXFP4 layout (MOE_W_MXFP4; what moe_expert_ffn reads): the same
 *     codes and scales regrouped into 16-row x 128-column blocks. Block
 *     (rb, s) of a matrix with K columns (nslab = K/128) holds rows
 *     16rb..16rb+15, columns 128s..128s+127:
 *       codes : 1024 bytes at (rb*nslab + s)*1024; bytes 16l..16l+15 are the
 *               32 codes of row 16rb + l%16, columns 128s + 32(l/16) + 0..31
 *               (even element in the low nibble);
 *       scales: 64 bytes at (rb*nslab + s)*64; byte l is the scale of row
 *               16rb + l%16, columns 128s + 32(l/16) + 0..31.
 *     Sizes equal the interchange layout's. Requires H and I to be multiples
 *     of 128.
 *   MOE_W_NVFP4 (aimodeling.com/en page, "Reported Numbers and Ecosystem
 *     Position", lists NVFP4 among the weight formats): value = E2M1 code x
 *     E4M3 block scale x one fp32 scale per matrix; one E4M3 scale per 16
 *     consecutive elements of a row. Interchange layout: codes as MXFP4, then
 *     scales [rows][K/16] (one byte each), then the matrix's fp32 scale in 16
 *     bytes (the scale pointer s13 / s2 points at the block scales; the fp32
 *     scale sits at s + rows*K/16). Kernel layout: codes as the kernel MXFP4
 *     layout; block scales 128 bytes per block at (rb*nslab + s)*128, bytes
 *     2l and 2l+1 holding the scales of columns 128s + 32(l/16) + 0..15 and
 *     + 16..31 of row 16rb + l%16; the fp32 scale stays at s + rows*K/16.
 *   MOE_W_FP8 (same page, FP8): value = E4M3 code x one fp32 scale per matrix.
 *     Interchange layout: rows of one-byte codes, then the fp32 scale in 16
 *     bytes (s13 / s2 point at it). Kernel layout: 2048-byte blocks at
 *     (rb*nslab + s)*2048; bytes 32l..32l+31 are row 16rb + l%16, columns
 *     128s + 32(l/16) + 0..31.
 *   E4M3 is the OCP 8-bit format with 4 exponent bits (bias 7) and 3 mantissa
 *   bits, no infinities, NaN = S.1111.111, largest finite 448.
 *   MOE_W_BF16: rows of bf16, row-major; scale pointers are ignored.
 * All weight matrix starts must be 16-byte aligned.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,        /* bad argument (size, null pointer, small workspace) */
    MOE_ENOMEM = -2,        /* not enough cache slots / host memory */
    MOE_EHIP = -3,          /* a HIP call failed; see moe_last_hip_error() */
    MOE_EUNSUPPORTED = -4,  /* valid request the library does not handle */
    MOE_EBUSY = -5          /* resource in use */
} moe_err;

typedef enum { MOE_W_BF16 = 0, MOE_W_MXFP4 = 1, MOE_W_NVFP4 = 2, MOE_W_FP8 = 3 } moe_wfmt;

/* One expert's weights. w13/w2 point to the codes (MXFP4, NVFP4, FP8) or the
 * bf16 values; s13/s2 point to the scale section of each matrix: E8M0 block
 * scales (MXFP4), E4M3 block scales followed by the fp32 matrix scale (NVFP4),
 * or the fp32 matrix scale alone (FP8); ignored for bf16. */
typedef struct {
    const void *w13;
    const uint8_t *s13;
    const void *w2;
    const uint8_t *s2;
} moe_expert_w;

/* Human-readable text for a moe_err. Never NULL. */
const char *moe_strerror(int err);
/* HIP error code of the last MOE_EHIP returned on this host thread. */
int moe_last_hip_error(void);

/*
 * moe_route -- router: top-k expert choice and mixing weights per token.
 *
 * Logits come either from logits_in [T][E] fp32, or (when logits_in is NULL)
 * from the router gate: logit[t][e] = sum_h x[t][h] * wg[e][h] over bf16 x
 * [T][H] and wg [E][H], formed in fp32 in a fixed order (lane l of 64 sums,
 * in ascending h, the products of the 8-element chunks c with c mod 64 == l;
 * the 64 partial sums are then combined by a butterfly with partner distances
 * 32,16,8,4,2,1), so that the choice of experts is reproducible bit for bit.
 * logits_out [T][E] (optional) receives the logits used.
 *
 * Selection: the k largest logits per token, in descending order; equal
 * logits are taken lower expert index first. topk_ids [T][k] int32.
 * Weights topk_w [T][k] fp32:
 *   renormalize != 0: w_j = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0)
 *                     (softmax over all E, renormalised over the k chosen)
 *   renormalize == 0: w_j = exp(l_j - l_max) / sum_{e<E} exp(l_e - l_max)
 * Requires 1 <= k <= min(E, 64), E <= 1024, T >= 0, H % 8 == 0 for the gate.
 * Logits must be finite (non-finite logits give unspecified routing).
 */
int moe_route(const uint16_t *x_bf16, const uint16_t *wg_bf16, const float *logits_in,
              float *logits_out, int T, int H, int E, int k, int renormalize,
              int32_t *topk_ids, float *topk_w, void *stream);

/*
 * moe_permute -- group the T*k token pairs by expert (stable counting sort).
 *
 * offsets [E+1]: offsets[e] = number of pairs routed to experts < e,
 *                offsets[E] = T*k (pairs of expert e are rows
 *                offsets[e] .. offsets[e+1]-1 of sorted order);
 * sorted_pair [T*k]: sorted_pair[offsets[e] + r] = the r-th pair, in
 *                ascending p, routed to expert e;
 * pair_row [T*k]: inverse, pair_row[sorted_pair[r]] = r.
 * ws: device workspace of at least the permute size from moe_workspace_size.
 * Requires E <= 512. Ids outside [0, E) are skipped (not counted; their
 * pair_row entry is left unwritten), so offsets[E] < T*k flags them.
 * T = 0 writes offsets only.
 */
int moe_permute(const int32_t *topk_ids, int T, int k, int E, int32_t *offsets,
                int32_t *sorted_pair, int32_t *pair_row, void *ws, size_t ws_bytes,
                void *stream);

/*
 * moe_route_permute -- moe_route followed by moe_permute, with the same
 * arguments and results as the two calls. For T <= 16 with the gate computed
 * here, or T <= 8 with logits_in given (and E <= 512), both run in one
 * single-workgroup kernel that keeps the chosen ids on chip (up to 64 pairs
 * one wavefront ranks them in registers); larger batches make the two calls.
 * ws / ws_bytes as for moe_permute.
 */
int moe_route_permute(const uint16_t *x_bf16, const uint16_t *wg_bf16, const float *logits_in,
                      float *logits_out, int T, int H, int E, int k, int renormalize,
                      int32_t *topk_ids, float *topk_w, int32_t *offsets, int32_t *sorted_pair,
                      int32_t *pair_row, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_expert_ffn -- grouped SwiGLU expert FFN over the permuted pairs.
 *
 * For every row r of sorted order, with e its expert (offsets[e] <= r <
 * offsets[e+1]) and t = sorted_pair[r] / k its token:
 *   g = W1_e x_t, u = W3_e x_t, a = silu(g) * u (silu(g) = g / (1 + e^-g)),
 *   y[sorted_pair[r]] = W2_e a.
 * y [T*k][H] is written in pair order (row p = t*k + j), bf16 (y_is_fp32 = 0)
 * or fp32. Accumulation is fp32. Between the two contractions the activation
 * a is rounded to bf16 (weight-streaming kernels), or, in the tiled kernels
 * (MXFP4, chosen when experts see many rows), x and a enter the block-scaled
 * FP8 x FP4 matrix cores as two E4M3 terms hi + lo with one E8M0 scale per
 * 32 elements: |hi + lo - v| <= 2^-8 |v| + 2^-22 max|block| for every v.
 * experts: device array [E] of moe_expert_w; entries of experts that receive
 * no pair are never read. x_bf16 [T][H]. fmt: MOE_W_MXFP4, MOE_W_NVFP4 or
 * MOE_W_FP8 (kernel layouts, H and I multiples of 128) or MOE_W_BF16 (H and
 * I multiples of 32). NVFP4 always runs the weight-streaming kernels (the
 * tiled kernels' matrix-core instruction takes only E8M0 block scales over 32
 * elements); FP8 runs either, the tiled kernels with unit block scales. The
 * weights enter the products as code x block scale, which is exact, and the
 * per-matrix fp32 scale multiplies the fp32 sums. Weight-streaming FP8 products
 * are bf16 x bf16 as for the other formats; NVFP4 products are fp16 x fp16:
 * x and the activation are carried in fp16 (exact for bf16 x with magnitude
 * in [2^-14, 65504]), so NVFP4 layers need activations below 65504.
 * ws: device workspace of at least the ffn size from moe_workspace_size.
 * Requires E <= 512.
 * The shared (always-on) expert is this call with E = 1, k = 1,
 * sorted_pair = 0..T-1 and offsets = {0, T}; moe_expert_ffn_shared runs it
 * inside the routed launches instead where the weight-streaming kernels run.
 */
int moe_expert_ffn(const uint16_t *x_bf16, const int32_t *sorted_pair, const int32_t *offsets,
                   const moe_expert_w *experts, int fmt, int T, int k, int H, int I, int E,
                   void *y, int y_is_fp32, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_expert_ffn_shared -- moe_expert_ffn for the routed experts together with
 * the always-on shared expert, in the same launches (a separate shared-expert
 * launch does not overlap a routed one that fills the device):
 *   y[p] for p < T*k as moe_expert_ffn; y[T*k + t] = W2_s (silu(W1_s x_t) *
 *   (W3_s x_t)) with the shared expert's weights `shared` (device pointer to
 *   one moe_expert_w, same format and sizes as the routed experts).
 * Weight-streaming kernels: the shared expert enters as more experts of the
 * launch, its T tokens in blocks of 16 when no routed expert has more than 16
 * rows (every block reads the shared weights; blocks run close together, so
 * the repeats mostly hit the caches), else as one. Tiled kernels: it is
 * expert E of the token-tile map, its rows the tokens in order.
 * y: [T*k + T][H], bf16 (y_is_fp32 = 0) or fp32; moe_combine takes rows T*k ..
 * as its y_shared. Numerics as moe_expert_ffn's (on the path it chooses).
 * ws: device workspace of at least the ffn size from moe_workspace_size(T,
 * k + 1, H, I, E) (the activation holds the shared expert's rows too).
 * Errors as moe_expert_ffn (shared == NULL is MOE_EINVAL).
 */
int moe_expert_ffn_shared(const uint16_t *x_bf16, const int32_t *sorted_pair,
                          const int32_t *offsets, const moe_expert_w *experts,
                          const moe_expert_w *shared, int fmt, int T, int k, int H, int I, int E,
                          void *y, int y_is_fp32, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_expert_ffn_noalloc -- moe_expert_ffn without a caller workspace, for
 * callers that cannot allocate device memory (code under stream/graph
 * capture, tight serving loops, harnesses that forbid allocation).
 * Arguments, results, numerics and errors as moe_expert_ffn, minus ws and
 * ws_bytes: the workspace is a device array of MOE_FFN_NOALLOC_MAX_WS bytes
 * inside this library, one per device, reserved when the library's kernels
 * are loaded on that device and held until the process ends. The call itself
 * allocates nothing. Requests whose workspace (the ffn size from
 * moe_workspace_size) exceeds MOE_FFN_NOALLOC_MAX_WS return MOE_ENOMEM before
 * any device work. The array is used on the calling thread's current device
 * (stream must belong to it). All calls on one device share the array: calls
 * whose work may overlap on the device (different streams without ordering
 * between them) race and give undefined results; calls ordered on one stream
 * are safe. Nothing in the array needs to start at a particular value.
 */
#define MOE_FFN_NOALLOC_MAX_WS ((size_t)64 << 20)
int moe_expert_ffn_noalloc(const uint16_t *x_bf16, const int32_t *sorted_pair,
                           const int32_t *offsets, const moe_expert_w *experts, int fmt, int T,
                           int k, int H, int I, int E, void *y, int y_is_fp32, void *stream);

/*
 * moe_combine -- weighted sum of each token's k expert outputs.
 *   out[t][n] = bf16_rne( sum_{j<k} topk_w[t][j] * y[t*k+j][n] + y_shared[t][n] )
 * summed in fp32 with j ascending; y_shared [T][H] (same dtype as y) is
 * optional (NULL = no shared expert) and added with weight 1.
 * out_bf16 [T][H]. Requires H % 8 == 0.
 */
int moe_combine(const void *y, int y_is_fp32, const float *topk_w, const void *y_shared, int T,
                int k, int H, uint16_t *out_bf16, void *stream);

/*
 * moe_expert_ffn_combine -- the expert FFN followed by the weighted combine:
 *   moe_expert_ffn (shared == NULL) or moe_expert_ffn_shared into y_bf16,
 *   then out_bf16[t] = moe_combine of those rows (the shared expert's rows
 *   T*k .. T*k + T - 1 as y_shared), both with bf16 y.
 * The combine is the second half of the layer's output step (the pages'
 * routed experts are mixed by the router's weights; winzheng.com page, "Why
 * Now of All Times"). At a handful of rows (T*k plus the shared expert's T
 * at most 15, block-scaled weights, the weight-streaming kernels)
 * the down projection and the combine run as one launch: each workgroup
 * computes 16 output columns of every routed row and sums each token's rows
 * for those columns. out is moe_combine's expression on the bf16 y this call
 * writes (fp32, j ascending), and y is within the tolerance of moe_expert_ffn
 * (the down projection's K order differs, so y need not equal
 * moe_expert_ffn's bit for bit). Otherwise the call is exactly the two calls.
 * y_bf16: [T*k][H], or [T*k + T][H] with the shared expert; out_bf16 [T][H];
 * topk_w [T][k] (moe_route's weights). ws: the ffn workspace of
 * moe_workspace_size(T, k, ...), or (T, k + 1, ...) with the shared expert.
 * Errors as moe_expert_ffn; topk_w, y_bf16 and out_bf16 must not be NULL.
 */
int moe_expert_ffn_combine(const uint16_t *x_bf16, const int32_t *sorted_pair,
                           const int32_t *offsets, const moe_expert_w *experts,
                           const moe_expert_w *shared, int fmt, int T, int k, int H, int I, int E,
                           const float *topk_w, uint16_t *y_bf16, uint16_t *out_bf16, void *ws,
                           size_t ws_bytes, void *stream);

/*
 * moe_permute_ffn_combine -- moe_permute followed by moe_expert_ffn_combine
 * (the router's ids in; the permutation, y and the layer output out), with
 * the same results as the two calls: offsets, sorted_pair and pair_row
 * bitwise, y and out as moe_expert_ffn_combine gives them.
 *
 * The routed experts are found from the ids (winzheng.com page, "Why Now of
 * All Times": a few of the layer's experts per token), so the grouping by
 * expert can happen where the experts' weights are first needed. For MXFP4
 * weights with E <= 256 and up to 512 pairs on the weight-streaming kernels,
 * the gate/up launch derives the expert offsets and each block's pairs from
 * the ids itself (in LDS), one of its workgroups writes the permutation out
 * for the down projection (with the combine in the same launch at up to 15
 * activation rows, as in moe_expert_ffn_combine) and the combine, so no
 * permutation launch runs. Otherwise the two calls run; the permutation's
 * workspace, where it needs one, is ws. T = 0 writes offsets only (all zero).
 * ws / ws_bytes as for moe_expert_ffn_combine. Errors as moe_expert_ffn_combine;
 * topk_ids, sorted_pair and pair_row must not be NULL for T > 0.
 */
int moe_permute_ffn_combine(const uint16_t *x_bf16, const int32_t *topk_ids,
                            const float *topk_w, const moe_expert_w *experts,
                            const moe_expert_w *shared, int fmt, int T, int k, int H, int I,
                            int E, int32_t *offsets, int32_t *sorted_pair, int32_t *pair_row,
                            uint16_t *y_bf16, uint16_t *out_bf16, void *ws, size_t ws_bytes,
                            void *stream);

/* Bytes of the barrier buffer moe_layer_fused takes. */
#define MOE_LAYER_SYNC_BYTES 8192

/*
 * moe_layer_fused -- the whole layer from given router logits in one launch,
 * for a handful of tokens: moe_route (logits given, no logits written), then
 * moe_permute_ffn_combine, with the same results: topk_ids, topk_w, offsets,
 * sorted_pair and pair_row bitwise, y and out as moe_expert_ffn_combine gives
 * them at these sizes.
 *
 * Batch-1 decoding is the pages' use case (winzheng.com page, "Why Now of All
 * Times": per token and layer a few routed experts out of hundreds); there
 * the layer's weight bytes take microseconds to stream while a chain of
 * dependent launches costs several microseconds per launch. Every workgroup
 * routes the tokens and derives the permutation itself, the gate/up tiles
 * are spread over all compute units, and the down projection + combine
 * workgroups request their weights before waiting at a grid barrier for the
 * activation rows.
 *
 * Taken for MXFP4 weights, 1 <= T <= 8, T*k (+ T with the shared expert) <=
 * 31 rows, E <= 256 and (H, I) one of (1024, 512), (2048, 512), (2048, 768),
 * (4096, 768), (4096, 2048), on a device whose compute units hold one
 * workgroup each for all H/16 down-projection workgroups (a multiple of 16
 * compute units, at least H/16); otherwise MOE_EUNSUPPORTED before any
 * device work (use moe_route + moe_permute_ffn_combine).
 *   logits [T][E] fp32; renormalize as moe_route; topk_ids/topk_w [T][k] out;
 *   offsets [E+1], sorted_pair and pair_row [T*k] out; y_bf16, out_bf16, ws
 *   and ws_bytes as moe_permute_ffn_combine.
 *   sync: MOE_LAYER_SYNC_BYTES of device memory (8-byte aligned) holding the
 *     launch's barrier counters. Zero it before the first call that uses it
 *     (e.g. one hipMemset); the calls keep it consistent from then on (its
 *     counters only grow). The 64-bit word at byte offset 4224 becomes
 *     nonzero if a barrier wait ran out (about a second), in which case that
 *     call's outputs are not valid; this happens only if the launch's
 *     workgroups cannot all be resident at once. Calls on one sync buffer must not overlap in time
 *     (one stream, or ordered streams); calls that may run side by side need
 *     their own sync buffers and workspaces, and two such launches on one
 *     device may each hold compute units the other waits for: run them on one
 *     stream.
 * Errors: MOE_EINVAL for NULL pointers, sizes out of range or a workspace too
 * small; MOE_EHIP if the launch fails.
 */
int moe_layer_fused(const uint16_t *x_bf16, const float *logits, const moe_expert_w *experts,
                    const moe_expert_w *shared, int fmt, int T, int k, int H, int I, int E,
                    int renormalize, int32_t *topk_ids, float *topk_w, int32_t *offsets,
                    int32_t *sorted_pair, int32_t *pair_row, uint16_t *y_bf16,
                    uint16_t *out_bf16, void *ws, size_t ws_bytes, void *sync, void *stream);

/*
 * moe_pack_mxfp4 -- convert n expert blobs from the interchange MXFP4 layout
 * to the kernel layout (see the top of this file). src and dst are device
 * buffers of n blobs spaced src_stride / dst_stride bytes apart; within a blob
 * the four sections sit at the byte offsets lay_w13, lay_s13, lay_w2, lay_s2
 * in both. Sizes are unchanged. src and dst must not overlap. H and I must
 * be multiples of 128.
 */
int moe_pack_mxfp4(const void *src, void *dst, int n, size_t src_stride, size_t dst_stride,
                   int H, int I, size_t lay_w13, size_t lay_s13, size_t lay_w2, size_t lay_s2,
                   void *stream);

/*
 * moe_pack_weights -- moe_pack_mxfp4 for any of MOE_W_MXFP4, MOE_W_NVFP4 and
 * MOE_W_FP8: interchange -> kernel layout of n blobs (same arguments; the
 * per-matrix fp32 scales are copied as they are).
 */
int moe_pack_weights(int fmt, const void *src, void *dst, int n, size_t src_stride,
                     size_t dst_stride, int H, int I, size_t lay_w13, size_t lay_s13,
                     size_t lay_w2, size_t lay_s2, void *stream);

/* Device workspace bytes needed by moe_permute and moe_expert_ffn for these
 * sizes (host call, no device work). Either output pointer may be NULL. */
int moe_workspace_size(int T, int k, int H, int I, int E, size_t *permute_bytes,
                       size_t *ffn_bytes);

/* Tuning and diagnostic knobs (process-wide).
 *   MOE_OPT_FFN_PATH: 0 = choose by size (default), 1 = force the decode
 *                     (weight-streaming) kernels, 2 = force the prefill
 *                     (tiled matrix-core) kernels.
 *   MOE_OPT_TIMING:   1 = launch every kernel of the library through
 *                     hipExtLaunchKernel with two events that take the
 *                     dispatch's own start and end times on the launch's
 *                     stream (do not use under graph capture); 0 = off.
 *                     Setting it clears the accumulated timings.
 *   MOE_OPT_DEC_SPLIT: weights of the weight-streaming kernels' split of the
 *                     tiles over their persistent workgroups: workgroup i
 *                     takes a contiguous share proportional to
 *                     1 - ws * (i / C) - wp * (i % C) / C, C = compute units
 *                     (later-dispatched workgroups receive their first data
 *                     later). Four bytes, each in units of 1/256 and below
 *                     128: stage 1 ws, stage 1 wp, stage 2 ws, stage 2 wp
 *                     (low byte first); -1 restores the default.
 *   MOE_OPT_CACHE_FAULT: test knob: n > 0 makes the n-th expert-cache copy
 *                     from now fail without being issued (the prefetch call
 *                     returns MOE_EHIP as for a failed hipMemcpyAsync); 0 = off.
 *   MOE_OPT_CACHE_DELAY_US: test knob: every prefetch that copies first holds
 *                     its copy stream this many microseconds (a host function
 *                     that sleeps), as a slow link would; 0 = off.
 *   MOE_OPT_CACHE_THROTTLE_MBS: test knob: every prefetch that copies also
 *                     holds its copy stream for (bytes it copies) / (value
 *                     MB/s) before the copies, so the link looks slower (rate
 *                     1 / (1/value + 1/link)); 0 = off.
 *   MOE_OPT_PRE_GROUP: consecutive weight tiles one workgroup of the tiled
 *                     kernels runs with its copy ring kept going (fewer
 *                     workgroup prologues): gate/up count in the low byte,
 *                     down count in the next (1..16 each; rounded down to a
 *                     divisor of the tiles per expert); -1 restores the default. */
enum { MOE_OPT_FFN_PATH = 1, MOE_OPT_TIMING = 2, MOE_OPT_DEC_SPLIT = 3, MOE_OPT_CACHE_FAULT = 4,
       MOE_OPT_CACHE_DELAY_US = 5, MOE_OPT_CACHE_THROTTLE_MBS = 6, MOE_OPT_PRE_GROUP = 7 };
int moe_set_option(int option, int value);
int moe_get_option(int option);

/* Kernel ids 0 .. (number of kernels - 1); NULL past the last. */
const char *moe_kernel_name(int kernel_id);
/* Launches of kernel_id timed since MOE_OPT_TIMING was last set, and their
 * summed durations in milliseconds (waits for the recorded events). */
int moe_timing_query(int kernel_id, long long *launches, double *total_ms);

/* ---------------------------------------------------------------------------
 * Measurement helpers (not part of the layer): the references the layer's
 * kernels are compared with in a benchmark.
 *
 * moe_micro_read -- read `bytes` (a multiple of 16) of the device buffer buf
 * (16-byte aligned) once, with `grid` workgroups of 256 threads taking 64 KB
 * chunks in turn, 16-byte non-temporal loads. sink: device word written only
 * in a case that does not occur (keeps the loads). Time it with events.
 *
 * moe_micro_mfma -- `grid` workgroups of four wavefronts each issue `iters` x 4
 * independent matrix-core instructions: kind 0 = bf16 32x32x16, kind 1 =
 * block-scaled 16x16x128 with an E2M1 A and an E4M3 B operand. *flops (host,
 * optional) receives the FLOPs of the launch. sink as above.
 */
int moe_micro_read(const void *buf, size_t bytes, int grid, void *sink, void *stream);
int moe_micro_mfma(int kind, int grid, int iters, void *sink, double *flops, void *stream);

/* ---------------------------------------------------------------------------
 * Expert cache: a pool of device slots holding expert blobs copied from pinned
 * host memory, with a per-layer device table of moe_expert_w that points into
 * the slots. The host keeps the least-recently-used order over (layer,
 * expert) keys and evicts the least recently used unpinned slot on a miss.
 * Copies are hipMemcpyAsync from pinned host memory on the copy stream given
 * at reserve time, so they overlap with compute on other streams.
 */
typedef struct moe_cache moe_cache;

/*
 * expert_cache_reserve -- create a cache over a caller-owned device pool.
 * pool: device buffer of pool_bytes (owned by the caller; must outlive the
 *       cache); it is cut into floor(pool_bytes / slot_bytes) slots, where
 *       slot_bytes is expert_bytes rounded up to 256.
 * host_src: (host) array [n_layers * n_experts] of pointers to each expert's
 *       blob in pinned host memory (entry layer*n_experts + e); the array is
 *       copied, the blobs must outlive the cache.
 * lay_*: byte offsets of w13/s13/w2/s2 inside a blob (the table entries are
 *       slot + offset).
 * copy_stream: stream for the host-to-device copies.
 * Returns MOE_ENOMEM if the pool holds fewer slots than n_experts.
 */
int expert_cache_reserve(moe_cache **cache, void *pool, size_t pool_bytes, size_t expert_bytes,
                         int n_layers, int n_experts, const void *const *host_src,
                         size_t lay_w13, size_t lay_s13, size_t lay_w2, size_t lay_s2,
                         void *copy_stream);

/*
 * expert_cache_prefetch -- make experts of one layer resident.
 * ids: (host) expert indices of `layer` to make resident (duplicates
 *      allowed); NULL means every expert of the layer.
 * Hits refresh the LRU order; each miss takes the least recently used slot
 * that no call since the previous prefetch has handed out, waits (on the copy
 * stream) for the compute work that last used it, and copies the blob into it
 * (free slots count as least recently used, the lowest index first; misses
 * whose blobs are adjacent in host memory and whose slots are adjacent share
 * one copy).
 * If a copy cannot be enqueued (MOE_EHIP), the misses enqueued before it are
 * resident (their copies are in flight; compute_stream waits for them), and
 * nothing else of the call takes effect: no hit is refreshed, no other slot
 * changes, the counters count only the enqueued copies. A failure at the
 * call's first copy therefore leaves the cache exactly as it was.
 * On return, compute_stream has been made to wait for this layer's copies and
 * table update, and *table_out (if not NULL) is the layer's device table
 * [n_experts] for moe_expert_ffn. Entries of experts not requested may be
 * stale and must not be read (moe_expert_ffn only reads experts with pairs).
 * Returns MOE_ENOMEM (cache unchanged) if more distinct misses are requested
 * than slots can be freed.
 */
int expert_cache_prefetch(moe_cache *cache, int layer, const int32_t *ids, int n,
                          void *compute_stream, const moe_expert_w **table_out);

/*
 * expert_cache_resize -- move the cache to a pool of another size at run time
 * (the expert-cache side of re-allocating device memory between the expert
 * cache and other uses without reloading weights).
 * new_pool: caller-owned device buffer of new_pool_bytes; either the current
 *       pool itself (shrink or grow in place: its first new_pool_bytes bytes)
 *       or a buffer that does not overlap the current pool.
 * The min(residents, new slot count) most recently used residents stay
 * resident, moved by device-to-device copies on the copy stream (a resident
 * keeps its slot index when it is below the new slot count, the others take
 * the lowest free indices, most recent first); the rest are dropped. LRU
 * order among the kept residents is unchanged; free slots become the least
 * recently used, the lowest index to be taken first. The copy stream first waits for
 * the work enqueued on compute_stream before this call; on return,
 * compute_stream waits for the copies and table updates.
 * Tables returned by earlier prefetch calls must not be read by compute
 * enqueued after this call (prefetch again). A separate old pool may be
 * released once compute_stream has passed this call.
 * moved (may be NULL): number of experts copied.
 * Returns MOE_ENOMEM if the new pool holds fewer slots than n_experts, and
 * MOE_EINVAL for a partial overlap, with the cache unchanged; after a HIP
 * error during the copies the cache stays on the old pool without the
 * residents that did not fit.
 */
int expert_cache_resize(moe_cache *cache, void *new_pool, size_t new_pool_bytes,
                        void *compute_stream, int *moved);

/*
 * expert_cache_bandwidth -- the host-to-device rate the cache's copies have
 * actually achieved (the pages' system keeps measuring the bandwidth it really
 * gets, winzheng.com page, "FreeToken's Three-Layer Mechanism"): an
 * exponentially weighted mean (weight 1/4 for the newest) of bytes / time over
 * the copies of completed prefetch calls, each call's copies timed by two
 * events on the copy stream (waits for free slots and any contention inside
 * the call count against the rate). *gbs = 0 until a call with copies has
 * completed; *samples = the calls folded in. Either pointer may be NULL.
 */
int expert_cache_bandwidth(moe_cache *cache, double *gbs, long long *samples);

/*
 * expert_cache_prefetch_qstar -- expert_cache_prefetch with the pages'
 * bandwidth-adaptive choice of the side that computes each expert (the q*
 * policy: GPU or host CPU by the bandwidth actually available; winzheng.com
 * page, "FreeToken's Three-Layer Mechanism"; aimodeling.com/en page, "Three
 * Engineering Cores").
 * ids, rows: (host) [n] requested experts of `layer` and the number of token
 * rows each has (duplicates add up). A resident expert stays on the device.
 * A missing one costs expert_bytes / rate on the link, or host_s_per_expert
 * + rows x host_s_per_row (seconds) on the host, plus host_s_fixed once if
 * the host takes any expert (its inputs read back, its rows sent), and both
 * sides work at the same time:
 * misses move to the host, fewest rows first, while the host's summed time
 * stays within the copy time left to the link. rate: link_gbs if > 0, else
 * expert_cache_bandwidth's (no expert goes to the host before it is known).
 * The device experts are then requested as by expert_cache_prefetch (same
 * results, errors and table); the host experts are not copied.
 * host_mask: (host) [n_experts] out: 1 for the experts to compute on the host
 * (with moe_cpu_expert_ffn from their host blobs), else 0; *n_host (may be
 * NULL) their number. On error host_mask is not written.
 */
int expert_cache_prefetch_qstar(moe_cache *cache, int layer, const int32_t *ids,
                                const int32_t *rows, int n, double host_s_fixed,
                                double host_s_per_expert, double host_s_per_row, double link_gbs,
                                void *compute_stream, const moe_expert_w **table_out,
                                uint8_t *host_mask, int *n_host);

/*
 * moe_permute_split -- (host arrays) moe_permute's result restricted to the
 * experts with host_mask[e] == 0, for moe_expert_ffn on the device: their rows
 * in the same order, the masked experts' counts zero (dev_offsets [E+1],
 * dev_sorted_pair [offsets[E]]); and the masked experts' pairs in sorted order
 * (host_pairs [offsets[E]], *n_host of them), for the host kernel and
 * moe_scatter_rows.
 */
int moe_permute_split(const int32_t *offsets, const int32_t *sorted_pair, int E,
                      const uint8_t *host_mask, int32_t *dev_offsets, int32_t *dev_sorted_pair,
                      int32_t *host_pairs, int *n_host);

/*
 * moe_cpu_expert_ffn -- (host) one expert's SwiGLU FFN on the host CPU, for the
 * experts the bandwidth-adaptive choice leaves on the host:
 *   y_rows[r] = W2 (silu(W1 x_r) * (W3 x_r)),  r < n,
 * x_rows [n][H] and y_rows [n][H] bf16 in host memory; the weights in host
 * memory in the kernel MXFP4 layout (fmt must be MOE_W_MXFP4; w13/s13/w2/s2 as
 * in moe_expert_w, e.g. a blob of the cache's pinned host store). fp32
 * accumulation; the activation is rounded to bf16 between the contractions.
 * threads: host threads (OpenMP; 0 = the default count). Synchronous.
 */
int moe_cpu_expert_ffn(int fmt, const void *w13, const uint8_t *s13, const void *w2,
                       const uint8_t *s2, int H, int I, const uint16_t *x_rows, int n,
                       uint16_t *y_rows, int threads);

/*
 * moe_scatter_rows -- dst row idx[r] = src row r for r < n (device arrays;
 * rows of row_bytes bytes, a multiple of 16; every idx[r] must index a row of
 * dst): the host-computed expert rows into y at their pairs.
 */
int moe_scatter_rows(const void *src, const int32_t *idx, int n, size_t row_bytes, void *dst,
                     void *stream);

/* expert_cache_evict -- drop experts of `layer` from the cache (NULL ids =
 * the whole layer). Their slots become free for later misses. */
int expert_cache_evict(moe_cache *cache, int layer, const int32_t *ids, int n);

/* Counters since reserve: hits, misses, bytes copied host-to-device. */
int expert_cache_stats(const moe_cache *cache, long long *hits, long long *misses,
                       long long *h2d_bytes);

/* Number of slots and the slot (or -1) holding (layer, expert). */
int expert_cache_slots(const moe_cache *cache);
int expert_cache_slot_of(const moe_cache *cache, int layer, int expert);

/* Release the cache's metadata (host and its device table). Synchronises the
 * copy stream first. The pool stays the caller's. */
int expert_cache_destroy(moe_cache *cache);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
