// Permutation of token pairs by expert: a stable counting sort.
//
// Each 1024-pair chunk is ranked without order-deciding atomics: within a
// wavefront, lanes holding the same expert are found by a ballot per id bit
// (a multisplit) and ranked by popcount of the lower lanes; the 16 wavefronts
// of a chunk are ordered by a per-expert prefix over their counts in LDS.
//   small path (T*k <= kSmallMax): one workgroup does histogram, scan and scatter;
//   large path: per-chunk ranks + histograms, one column scan, one scatter.
#include "route_dev.hpp"

namespace moe {

constexpr int kChunk = 1024;            // pairs per chunk (one per thread)
constexpr int kWavesPerChunk = kChunk / kWave;
constexpr int kMaxE = 512;
constexpr int kSmallMax = 4 * kChunk;   // pairs handled by the one-workgroup kernel
constexpr int kFusedMaxT = 16;          // fused router + permutation, gate computed in the kernel
constexpr int kFusedMaxLogitsT = 8;     // fused router + permutation, logits given

// Multisplit rank of this lane's expert e within its wavefront. Returns the
// number of lower lanes with the same e; *count = lanes with the same e.
__device__ __forceinline__ int wave_rank(bool valid, int e, int nbits, int *count) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    *count = __popcll(m);
    return __popcll(m & lanemask_lt());
}

__device__ __forceinline__ int id_bits(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

// Ranks the chunk's pairs. wcnt [16][E] must be zero on entry; on return
// wcnt[w][e] holds the number of pairs of expert e in waves < w of the chunk
// and tot[e] the chunk's count of e. Returns the lane's rank within its
// expert in the chunk (valid lanes only).
__device__ int chunk_rank(bool valid, int e, int E, int nbits, int *wcnt, int *tot) {
    const int w = threadIdx.x / kWave;
    int cnt;
    const int r = wave_rank(valid, e, nbits, &cnt);
    if (valid && r == 0) wcnt[w * E + e] = cnt;
    __syncthreads();
    for (int x = threadIdx.x; x < E; x += blockDim.x) {
        int run = 0;
        for (int ww = 0; ww < kWavesPerChunk; ++ww) {
            const int c = wcnt[ww * E + x];
            wcnt[ww * E + x] = run;
            run += c;
        }
        tot[x] = run;
    }
    __syncthreads();
    return valid ? wcnt[w * E + e] + r : 0;
}

// Block-wide exclusive scan of in[0..E) into out[0..E], out[E] = total.
// 1024 threads, E <= 1024. scratch: >= 32 ints.
__device__ void block_exclusive_scan(const int *in, int *out, int E, int *scratch) {
    const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
    int v = tid < E ? in[tid] : 0;
    int incl = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) scratch[w] = incl;
    __syncthreads();
    if (w == 0) {
        int s = lane < kWavesPerChunk ? scratch[lane] : 0;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int o = __shfl_up(s, d);
            if (lane >= d) s += o;
        }
        if (lane < kWavesPerChunk) scratch[16 + lane] = s;   // inclusive wave totals
    }
    __syncthreads();
    const int wave_base = w ? scratch[16 + w - 1] : 0;
    if (tid < E) out[tid] = wave_base + incl - v;
    if (tid == E - 1) out[E] = wave_base + incl;
    __syncthreads();
}

// Whole permutation of n <= kSmallMax pairs by one 1024-thread workgroup.
// `ids` may point to global memory or LDS; `lds` holds (19E + 33) ints.
__device__ void permute_block(const int32_t *ids, int n, int E, int32_t *__restrict__ offsets,
                              int32_t *__restrict__ sorted_pair, int32_t *__restrict__ pair_row,
                              int *lds) {
    int *cnt = lds;                       // [E]
    int *base = cnt + E;                  // [E+1]
    int *tot = base + E + 1;              // [E]
    int *scratch = tot + E;               // [32]
    int *wcnt = scratch + 32;             // [16][E]
    const int tid = threadIdx.x;
    const int nbits = id_bits(E);

    for (int x = tid; x < E; x += kChunk) cnt[x] = 0;
    for (int x = tid; x < kWavesPerChunk * E; x += kChunk) wcnt[x] = 0;
    __syncthreads();
    for (int p = tid; p < n; p += kChunk) {
        const int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    block_exclusive_scan(cnt, base, E, scratch);
    for (int x = tid; x <= E; x += kChunk) offsets[x] = base[x];

    for (int c0 = 0; c0 < n; c0 += kChunk) {
        const int p = c0 + tid;
        const int e = p < n ? ids[p] : -1;
        const bool valid = e >= 0 && e < E;
        const int r = chunk_rank(valid, e, E, nbits, wcnt, tot);
        if (valid) {
            const int pos = base[e] + r;
            sorted_pair[pos] = p;
            pair_row[p] = pos;
        }
        __syncthreads();
        for (int x = tid; x < E; x += kChunk) base[x] += tot[x];
        for (int x = tid; x < kWavesPerChunk * E; x += kChunk) wcnt[x] = 0;
        __syncthreads();
    }
}

__device__ __host__ constexpr size_t permute_block_lds_ints(int E) { return (size_t)19 * E + 33; }

__global__ __launch_bounds__(kChunk) void permute_small_kernel(
    const int32_t *__restrict__ ids, int n, int E, int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_pair, int32_t *__restrict__ pair_row) {
    extern __shared__ int lds[];
    permute_block(ids, n, E, offsets, sorted_pair, pair_row, lds);
}

// Router + permutation in one workgroup (T <= kFusedMaxT, or kFusedMaxLogitsT
// when logits are given): wavefront w routes token w; the chosen ids stay in
// LDS for the permutation. Beyond that the router's selection rounds (about 85
// dependent vector instructions per token and round) need more than one
// compute unit, and the separate router and permutation kernels win.
template <int VPL>
__global__ __launch_bounds__(kChunk) void route_permute_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg,
    const float *__restrict__ logits_in, float *__restrict__ logits_out, int T, int H, int E,
    int k, int renormalize, int32_t *__restrict__ topk_ids, float *__restrict__ topk_w,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_pair,
    int32_t *__restrict__ pair_row) {
    extern __shared__ int lds[];
    int *ids_lds = lds;                   // [T*k]
    int *plds = lds + T * k;
    const int w = threadIdx.x / kWave, lane = lane_id();
    for (int t = w; t < T; t += kWavesPerChunk) {
        const int id = route_token<VPL>(t, x, wg, logits_in, logits_out, H, E, k, renormalize,
                                        topk_ids, topk_w);
        if (lane < k) ids_lds[t * k + lane] = id;
    }
    __syncthreads();
    permute_block(ids_lds, T * k, E, offsets, sorted_pair, pair_row, plds);
}

// Router + permutation for tiny batches (at most 64 pairs, one wavefront per
// token): wavefront t routes token t; wavefront 0 then ranks the pairs in its
// lanes (lane p holds pair p): the multisplit rank within each expert, a
// histogram in LDS (one writer per expert), and the offsets by a wavefront
// scan with nine experts per lane (E <= 512, offsets[0..E]). Wavefront-local
// LDS writes and reads need no barrier: one wavefront's LDS operations run in
// order.
constexpr int kTinyPer = 9;             // experts per lane in the tiny kernel's scan
static_assert(kTinyPer * 64 >= kMaxE + 1, "tiny kernel scan must cover offsets[0..E]");
template <int VPL>
__global__ __launch_bounds__(kChunk) void route_permute_tiny_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg,
    const float *__restrict__ logits_in, float *__restrict__ logits_out, int T, int H, int E,
    int k, int renormalize, int32_t *__restrict__ topk_ids, float *__restrict__ topk_w,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_pair,
    int32_t *__restrict__ pair_row) {
    __shared__ int ids_lds[kWave];
    __shared__ int cnt[kTinyPer * kWave];   // histogram, then exclusive offsets
    const int w = threadIdx.x / kWave, lane = lane_id();
    const int n = T * k;
    if (w < T) {
        const int id = route_token<VPL>(w, x, wg, logits_in, logits_out, H, E, k, renormalize,
                                        topk_ids, topk_w);
        if (lane < k) ids_lds[w * k + lane] = id;
    }
    for (int e = threadIdx.x; e < kTinyPer * kWave; e += blockDim.x) cnt[e] = 0;
    __syncthreads();
    if (w != 0) return;
    const int e = lane < n ? ids_lds[lane] : -1;
    const bool valid = e >= 0 && e < E;
    int same;
    const int r = wave_rank(valid, e, id_bits(E), &same);
    if (valid && r == 0) cnt[e] = same;
    __builtin_amdgcn_wave_barrier();
    int c[kTinyPer], tot = 0;
#pragma unroll
    for (int i = 0; i < kTinyPer; ++i) {
        c[i] = cnt[kTinyPer * lane + i];
        tot += c[i];
    }
    int incl = tot;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    int base = incl - tot;
#pragma unroll
    for (int i = 0; i < kTinyPer; ++i) {
        const int ex = kTinyPer * lane + i;
        cnt[ex] = base;
        if (ex <= E) offsets[ex] = base;
        base += c[i];
    }
    __builtin_amdgcn_wave_barrier();
    if (valid) {
        const int pos = cnt[e] + r;
        sorted_pair[pos] = lane;
        pair_row[lane] = pos;
    }
}

// Large path, pass 1: per-chunk ranks and histograms.
__global__ __launch_bounds__(kChunk) void permute_rank_kernel(
    const int32_t *__restrict__ ids, int n, int E, int32_t *__restrict__ hist /*[nb][E]*/,
    int32_t *__restrict__ lrank /*[n]*/) {
    extern __shared__ int lds[];
    int *tot = lds;                       // [E]
    int *wcnt = tot + E;                  // [16][E]
    const int tid = threadIdx.x;
    for (int x = tid; x < kWavesPerChunk * E; x += kChunk) wcnt[x] = 0;
    __syncthreads();
    const int p = blockIdx.x * kChunk + tid;
    const int e = p < n ? ids[p] : -1;
    const bool valid = e >= 0 && e < E;
    const int r = chunk_rank(valid, e, E, id_bits(E), wcnt, tot);
    if (valid) lrank[p] = r;
    for (int x = tid; x < E; x += kChunk) hist[(size_t)blockIdx.x * E + x] = tot[x];
}

// Large path, pass 2 (one workgroup): per expert, exclusive prefix over the
// chunks; offsets by a scan of the expert totals; hist becomes the scatter base.
// P = 1024 / E threads share an expert's column: each sums a contiguous run of
// chunks (independent loads), the runs' totals are prefixed in LDS, then each
// thread rewrites its run.
__global__ __launch_bounds__(kChunk) void permute_scan_kernel(int nb, int E,
                                                              int32_t *__restrict__ hist,
                                                              int32_t *__restrict__ offsets) {
    __shared__ int tot[kMaxE];
    __shared__ int off[kMaxE + 1];
    __shared__ int scratch[32];
    __shared__ int part[kChunk];
    const int tid = threadIdx.x;
    const int P = E < kChunk ? kChunk / E : 1;
    const int x = tid / P, p = tid - x * P;
    const int per = (nb + P - 1) / P;
    const int b0 = min(nb, p * per), b1 = min(nb, b0 + per);
    int sum = 0;
    if (x < E)
        for (int b = b0; b < b1; ++b) sum += hist[(size_t)b * E + x];
    part[tid] = sum;
    __syncthreads();
    int pre = 0;                       // this run's exclusive prefix within the column
    if (x < E)
        for (int q = 0; q < p; ++q) pre += part[x * P + q];
    if (x < E && p == P - 1) tot[x] = pre + sum;
    __syncthreads();
    block_exclusive_scan(tot, off, E, scratch);
    for (int y = tid; y <= E; y += kChunk) offsets[y] = off[y];
    if (x < E) {
        int run = off[x] + pre;
        for (int b = b0; b < b1; ++b) {
            const int c = hist[(size_t)b * E + x];
            hist[(size_t)b * E + x] = run;
            run += c;
        }
    }
}

// Large path, pass 3: scatter.
__global__ __launch_bounds__(kChunk) void permute_scatter_kernel(
    const int32_t *__restrict__ ids, int n, int E, const int32_t *__restrict__ hist,
    const int32_t *__restrict__ lrank, int32_t *__restrict__ sorted_pair,
    int32_t *__restrict__ pair_row) {
    const int p = blockIdx.x * kChunk + threadIdx.x;
    if (p >= n) return;
    const int e = ids[p];
    if (e < 0 || e >= E) return;
    const int pos = hist[(size_t)blockIdx.x * E + e] + lrank[p];
    sorted_pair[pos] = p;
    pair_row[p] = pos;
}

__global__ void permute_empty_kernel(int E, int32_t *offsets) {
    for (int x = threadIdx.x; x <= E; x += blockDim.x) offsets[x] = 0;
}

size_t permute_ws_bytes(long n, int E) {
    if (n <= kSmallMax) return 0;
    const long nb = (n + kChunk - 1) / kChunk;
    return (size_t)(nb * E + n) * sizeof(int32_t) + 256;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_permute(const int32_t *topk_ids, int T, int k, int E, int32_t *offsets,
                           int32_t *sorted_pair, int32_t *pair_row, void *ws, size_t ws_bytes,
                           void *stream) {
    if (T < 0 || k < 1 || E < 1 || E > kMaxE || !offsets) return MOE_EINVAL;
    const long n = (long)T * k;
    if (n > 0x7FFFFFFFL) return MOE_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (n == 0) {
        MOE_LAUNCH(K_PERM_EMPTY, permute_empty_kernel, dim3(1), dim3(256), 0, s, E, offsets);
        return check_launch();
    }
    if (!topk_ids || !sorted_pair || !pair_row) return MOE_EINVAL;
    if (n <= kSmallMax) {
        const size_t lds = permute_block_lds_ints(E) * sizeof(int);
        MOE_LAUNCH(K_PERM_SMALL, permute_small_kernel, dim3(1), dim3(kChunk), lds, s, topk_ids,
                                     (int)n, E, offsets, sorted_pair, pair_row);
        return check_launch();
    }
    if (ws_bytes < permute_ws_bytes(n, E) || !ws) return MOE_EINVAL;
    const int nb = (int)((n + kChunk - 1) / kChunk);
    int32_t *hist = (int32_t *)ws;
    int32_t *lrank = hist + (size_t)nb * E;
    const size_t lds1 = (size_t)(E + kWavesPerChunk * E) * sizeof(int);
    MOE_LAUNCH(K_PERM_RANK, permute_rank_kernel, dim3(nb), dim3(kChunk), lds1, s, topk_ids,
                                 (int)n, E, hist, lrank);
    int rc = check_launch();
    if (rc) return rc;
    MOE_LAUNCH(K_PERM_SCAN, permute_scan_kernel, dim3(1), dim3(kChunk), 0, s, nb, E, hist,
                                 offsets);
    rc = check_launch();
    if (rc) return rc;
    MOE_LAUNCH(K_PERM_SCATTER, permute_scatter_kernel, dim3(nb), dim3(kChunk), 0, s, topk_ids,
                                 (int)n, E, hist, lrank, sorted_pair, pair_row);
    return check_launch();
}

extern "C" int moe_route_permute(const uint16_t *x_bf16, const uint16_t *wg_bf16,
                                 const float *logits_in, float *logits_out, int T, int H, int E,
                                 int k, int renormalize, int32_t *topk_ids, float *topk_w,
                                 int32_t *offsets, int32_t *sorted_pair, int32_t *pair_row,
                                 void *ws, size_t ws_bytes, void *stream) {
    if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E || k > kWave || !offsets) return MOE_EINVAL;
    if (!logits_in && T > 0 && (!x_bf16 || !wg_bf16 || H < 8 || H % 8)) return MOE_EINVAL;
    const long n = (long)T * k;
    const int max_t = logits_in ? kFusedMaxLogitsT : kFusedMaxT;
    if (T == 0 || T > max_t || n > kSmallMax) {
        int rc = moe_route(x_bf16, wg_bf16, logits_in, logits_out, T, H, E, k, renormalize,
                           topk_ids, topk_w, stream);
        if (rc) return rc;
        return moe_permute(topk_ids, T, k, E, offsets, sorted_pair, pair_row, ws, ws_bytes,
                           stream);
    }
    if (!topk_ids || !topk_w || !sorted_pair || !pair_row) return MOE_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (n <= kWave) {
        // at most 64 pairs: one wavefront per token, the ranking in registers
        // (kTinyPer * 64 >= E + 1 offsets)
#define MOE_RPT(VPL)                                                                           \
    MOE_LAUNCH(K_ROUTE_PERMUTE, route_permute_tiny_kernel<VPL>, dim3(1), dim3(kWave * T), 0, s, \
               x_bf16, wg_bf16, logits_in, logits_out, T, H, E, k, renormalize, topk_ids,       \
               topk_w, offsets, sorted_pair, pair_row)
        if (E <= 64) MOE_RPT(1);
        else if (E <= 128) MOE_RPT(2);
        else if (E <= 256) MOE_RPT(4);
        else MOE_RPT(8);
#undef MOE_RPT
        return check_launch();
    }
    const size_t lds = ((size_t)n + permute_block_lds_ints(E)) * sizeof(int);
#define MOE_RP(VPL)                                                                            \
    MOE_LAUNCH(K_ROUTE_PERMUTE, route_permute_kernel<VPL>, dim3(1), dim3(kChunk), lds, s, x_bf16, \
                                 wg_bf16, logits_in, logits_out, T, H, E, k, renormalize,        \
                                 topk_ids, topk_w, offsets, sorted_pair, pair_row)
    if (E <= 64) MOE_RP(1);
    else if (E <= 128) MOE_RP(2);
    else if (E <= 256) MOE_RP(4);
    else MOE_RP(8);
#undef MOE_RP
    return check_launch();
}
