// The whole layer in one launch for a handful of tokens: router (softmax
// top-k from given logits), permutation, gate/up + SwiGLU, down projection
// and weighted combine.
//
// At one to four tokens (the single-user decoding the pages are built around:
// winzheng.com page, "Why Now of All Times", a few routed experts per token
// and layer) the layer moves a few tens of MB, and a chain of launches costs
// more than the bytes: every dependent launch adds its start-up, and each
// stage's weights are requested only once the stage before has ended. Here
// one persistent launch does it all:
//   1. every workgroup routes the T tokens itself (one wavefront per token,
//      the router kernel's device code, so ids and weights are the router's
//      bit for bit) and derives the permutation of the at most 31 pairs in
//      registers; workgroup 0 writes ids, weights and the permutation out;
//   2. gate/up tiles (16 gate + 16 up rows over K = H, K split over the 8
//      wavefronts, the weight-streaming kernel's tile code), split over all
//      workgroups, workgroups with down work taking fewer;
//   3. the workgroups with down work (one per 16 output columns) request
//      their W2 blocks of every active expert, then wait at a grid barrier
//      until every workgroup's activation rows are written; the down
//      projection and the combine then run as in the down + combine launch
//      (the activation rows staged in LDS in operand order, y and out
//      written; out is the combine's expression on the bf16 y).
// All workgroups must be resident at once: the grid is one workgroup per
// compute unit and the launch is refused unless the occupancy allows at least
// that many.
// The barrier's counters live in a caller buffer (zero before the first
// call; the counters only grow, so no call has to return them to zero); the
// wait is bounded (a flag reports a wait that ran out, and the call's
// results are then not valid).
#include <atomic>

#define MOE_DEC_SMALL_UNIT 1
#include "ffn_decode.hip"
#include "route_dev.hpp"

namespace moe {

constexpr int kFsWaves = kDcWaves;      // 8 wavefronts per workgroup
constexpr int kFsMaxRows = 31;          // activation rows (T*k, + T shared)
constexpr int kFsVpl = 4;               // logits per lane: E <= 256
constexpr unsigned kFsSpinLimit = 1u << 21;

// Barrier state in the caller's sync buffer: 64-bit words, one per 128-byte
// line (so that the groups' atomics and polls use separate lines):
//   line g < 16        arrivals of group g (workgroups b with b % 16 == g),
//                      counted over all calls;
//   line 16            groups complete, counted over all calls;
//   line 17 + g        release word of group g: the number of calls whose
//                      arrivals are complete;
//   line 33            set when a wait ran out.
// A call's arrivals are all counted before the next call's begin (calls on
// one buffer are ordered), so call j is the one whose arrivals in group g
// are j * size .. (j + 1) * size - 1, and its release is the value j + 1.
constexpr int kFsGroups = 16;
constexpr int kSyncLine = 16;           // 64-bit words per 128-byte line
constexpr int kSyncTop = kFsGroups, kSyncRel = kFsGroups + 1, kSyncTimeout = 2 * kFsGroups + 1;
static_assert((kSyncTimeout + 1) * kSyncLine * 8 <= MOE_LAYER_SYNC_BYTES, "sync buffer size");

struct FsArgs {
    const float *logits;     // [T][E] router logits
    int32_t *topk_ids;       // [T][k] out
    float *topk_w;           // [T][k] out
    int32_t *pair_row;       // [T*k] out
    uint16_t *out;           // [T][H] out
    uint64_t *sync;          // barrier state (MOE_LAYER_SYNC_BYTES)
    int T, renorm, nrows;    // nrows: T*k (+ T with the shared expert)
    int nd2;                 // workgroups with down + combine work (H / 16)
};

// Weighted split of the gate/up tiles: workgroup i < nd2 also streams the W2
// blocks of its 16 output columns (d tiles' worth of bytes), so it takes
// d tiles fewer, down to none. Returns the first tile of workgroup b.
__device__ __forceinline__ int fs_split(int b, int G, int nd2, int total, float d) {
    if (b >= G) return total;
    float sd = 1.0f, so = 1.0f;
    if (G > nd2) {
        const float tgt = ((float)total + (float)nd2 * d) / (float)G;
        sd = tgt - d;
        so = tgt;
        if (sd < 0.0f) {
            sd = 0.0f;
            so = (float)total / (float)(G - nd2);
        }
    }
    const float pb = (float)min(b, nd2) * sd + (float)max(b - nd2, 0) * so;
    const float pg = (float)nd2 * sd + (float)(G - nd2) * so;
    const int t = (int)((float)total * (pb / pg));
    return t < total ? t : total;
}

// The expert descriptions of one wavefront's down work (as dc_meta), with
// the offsets from the permutation in LDS.
template <int FMT, bool SH>
__device__ __forceinline__ DcMeta fs_meta(const DecArgs &A, const ShArgs &S, const ActiveSet &act,
                                          int wv, int n) {
    DcMeta d{0, 0, 0, 0, 1.0f};
    const int lane = lane_id();
    int e = 0, j = 0;
    for (int q = 0; q < n; ++q) {
        int jq;
        const int eq = act.template nth<SH>(wv + kFsWaves * q, A.E, jq);
        if (lane == q) {
            e = eq;
            j = jq;
        }
    }
    if (lane >= n) return d;
    const bool sh = SH && e == A.E;
    d.row0 = (sh ? S.T * A.k : act.loff[e]) + j * kPass;
    d.n_e = min(kPass, (sh ? S.T * (A.k + 1) : act.loff[e + 1]) - d.row0);
    const moe_expert_w *W = sh ? S.shared : A.experts + e;
    d.w = ld_global_u64(&W->w2);
    d.s = ld_global_u64(&W->s2);
    return d;
}

// The barrier's writes go to the device's coherence point without cache
// write-backs: the activation rows are stored written through (agent-scope
// atomic stores, in the tile code), the counters are agent-scope atomics and
// the release words are polled and the rows read back with device-coherent
// loads (measured faster than one acquire per workgroup followed by cached
// reads, and than cache write-backs at the arrivals). Order between a
// wavefront's own accesses comes from waiting for their completion (s_waitcnt, or the value an atomic
// returns) before the next is issued.
//
// Arrival of workgroup b (one lane, after its activation stores completed);
// returns the release value this call waits for.
__device__ __forceinline__ uint64_t fs_arrive(uint64_t *sync, int b, int G) {
    const int g = b % kFsGroups;
    const uint64_t size = (uint64_t)(G / kFsGroups);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the stores stay before the wait
    wait_vm<0>();
    const uint64_t old = __hip_atomic_fetch_add(&sync[g * kSyncLine], (uint64_t)1,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t call = old / size;
    if ((old + 1) % size == 0) {
        // last of its group in this call
        const uint64_t o2 = __hip_atomic_fetch_add(&sync[kSyncTop * kSyncLine], (uint64_t)1,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((o2 + 1) % kFsGroups == 0) {
            // last group: release every group
            for (int i = 0; i < kFsGroups; ++i)
                __hip_atomic_store(&sync[(kSyncRel + i) * kSyncLine], call + 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    return call + 1;
}

// Bounded wait for group g's release value to reach `want`.
__device__ __forceinline__ void fs_wait(uint64_t *sync, int b, uint64_t want) {
    const int g = b % kFsGroups;
    unsigned it = 0;
    while (__hip_atomic_load(&sync[(kSyncRel + g) * kSyncLine], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT) < want) {
        if (++it > kFsSpinLimit) {
            __hip_atomic_store(&sync[kSyncTimeout * kSyncLine], (uint64_t)1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(4);
    }
}


// ---- the permutation of at most 31 pairs, in registers -------------------
//
// The state init_ids + rank_ids build, for n <= 31 valid pairs (lane p holds
// pair p) and T <= 8 tokens, so every expert has at most 8 rows (one block):
// offsets of the active experts, each pair's stable rank (pairs of lower
// experts, then earlier pairs of its own), the active-expert blocks per group
// of 64 and the sorted pairs in this wavefront's LDS region (loff: [E + 1],
// the offsets of the active experts and of the expert after each; lsrt: [n]).
template <bool SH, int MAXN>
__device__ __forceinline__ int init_small(ActiveSet &act, const int32_t *rid, int n, int E,
                                          const ShArgs &S, int *wl) {
    const int lane = lane_id();
    act.loff = wl;
    act.lsrt = wl + 2 * E + 1;
    // every pair's id in registers (LDS broadcast reads; -1 past n), so that
    // the comparisons below stay in the vector unit: a lane read per pair
    // (vector -> scalar -> vector) made this part several times slower.
    // MAXN >= n: the unrolled length of the loops
    int idq[MAXN];
#pragma unroll
    for (int q = 0; q < MAXN; ++q) idq[q] = q < n ? rid[q] : -1;
    const int idp = lane < n ? rid[lane] : -1;
    int less = 0, same = 0, sbefore = 0;
#pragma unroll
    for (int q = 0; q < MAXN; ++q) {
        const int iq = idq[q];
        less += (iq >= 0 && iq < idp) ? 1 : 0;
        same += iq == idp ? 1 : 0;
        sbefore += (iq == idp && q < lane) ? 1 : 0;
    }
    const int rank = less + sbefore;
    if (lane < n) {
        act.loff[idp] = less;
        act.loff[idp + 1] = less + same;
        act.lsrt[rank] = lane;
    }
#pragma unroll
    for (int c = 0; c < kIdsChunks; ++c) act.idv[c] = c == 0 && lane < n ? idp : -1;
    act.count = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        act.incl[i] = 0;
        act.gtot[i] = 0;
        if (i * kWave < E) {
            const int e = i * kWave + lane;
            bool on = false;
#pragma unroll
            for (int q = 0; q < MAXN; ++q) on = on || idq[q] == e;
            const uint64_t mb = __ballot(on);
            act.incl[i] = __popcll(mb & (lanemask_lt() | (1ull << lane)));
            act.gtot[i] = __popcll(mb);
        }
        act.count += act.gtot[i];
    }
    act.routed = act.count;
    if constexpr (SH) {
        act.count += (S.T + kPass - 1) / kPass;
        act.sh_w = S.shared;
        act.sh_T = S.T;
    }
    return rank;
}

// Direct global -> LDS copy of 16 bytes per lane with a device-coherent load
// (past any stale line a cache may hold from an earlier call).
__device__ __forceinline__ void lds_dma16_coherent(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds((const MOE_GLOBAL void *)src, (MOE_LDS void *)dst, 16, 0,
                                     16 /* sc1 */);
}

// LDS (all dynamic): a head that lives through the launch (routed ids and
// weights, each row's pair, the router weight of each pair; 32 entries each),
// then one region used twice: by the gate/up part (the K-split partial sums,
// then the wavefronts' permutation regions) and, once those are dead (after
// the grid barrier), by the down + combine part (the activation rows in
// operand order, 4 KB per 16 rows and 128 columns, then the y columns).
constexpr size_t kFsHead = 4 * 32 * 4;
constexpr size_t kFsRed = (size_t)2 * (kFsWaves - 1) * 2 * 4 * kWave * 4;
__host__ __device__ constexpr size_t fs_phase1_bytes(int E, int n) {
    return kFsRed + (size_t)kFsWaves * ids_wave_ints(E, n) * 4;
}
__host__ __device__ constexpr size_t fs_phase3_bytes(int nrows, int ns2) {
    return (size_t)((nrows + 15) / 16) * ns2 * 4096 + (size_t)nrows * 16 * 4;
}
constexpr size_t kFsMaxLds = 160 * 1024;

template <int SPW1, int NS2, bool SH>
__global__ __launch_bounds__(kWave *kFsWaves) void ffn_small_kernel(DecArgs A1, DecArgs A2,
                                                                    ShArgs S, FsArgs F) {
    constexpr int FMT = MOE_W_MXFP4;
    extern __shared__ __attribute__((aligned(16))) uint8_t fs_lds[];
    const int lane = lane_id();
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int m = lane & 15, c = lane >> 4;
    const int tid = threadIdx.x;
    const int E = A1.E, k = A1.k, n = F.T * k;
    const int G = gridDim.x;

    const int wints = ids_wave_ints(E, n);
    int32_t *rid = reinterpret_cast<int32_t *>(fs_lds);        // [n] routed ids
    float *rw = reinterpret_cast<float *>(rid + 32);           // [n] weights
    int *spl = reinterpret_cast<int *>(rw + 32);               // [nrows] pair of each row
    float *wl = reinterpret_cast<float *>(spl + 32);           // [n] router weight of each pair
    uint8_t *reg = fs_lds + kFsHead;                           // the shared region
    auto &red = *reinterpret_cast<float (*)[2][kFsWaves - 1][2][4][kWave]>(reg);
    int *ids_lds = reinterpret_cast<int *>(reg + kFsRed);

    // 1. routing: wavefront t routes token t
    if (wv < F.T) {
        float v[1][kFsVpl];
        token_logits<kFsVpl>(wv, nullptr, nullptr, F.logits, 0, E, v[0]);
        int id[1];
        route_from_logits<kFsVpl, 1>(wv, 0, wv + 1, v, nullptr, E, k, F.renorm, rid, rw, id);
    }
    __syncthreads();
    ActiveSet act;
    // (shorter forms for up to 8 and 16 pairs: one or two tokens at k <= 8)
    int *const wl_ = ids_lds + wv * wints;
    const int rank = n <= 8    ? init_small<SH, 8>(act, rid, n, E, S, wl_)
                     : n <= 16 ? init_small<SH, 16>(act, rid, n, E, S, wl_)
                               : init_small<SH, kFsMaxRows>(act, rid, n, E, S, wl_);
    if (blockIdx.x == 0 && wv == 0) {
        // the router's and the permutation's outputs
        if (lane < n) {
            F.topk_ids[lane] = rid[lane];
            F.topk_w[lane] = rw[lane];
            F.pair_row[lane] = rank;
            const_cast<int32_t *>(A1.sorted_pair)[rank] = lane;
        }
        for (int e = lane; e <= E; e += kWave) {
            int o = 0;
            for (int q = 0; q < n; ++q) o += rid[q] < e ? 1 : 0;
            const_cast<int32_t *>(A1.offsets)[e] = o;
        }
    }

    // 2. gate/up tiles
    {
        const int total = act.count * A1.nrt;
        const float d = (float)act.count * (float)A1.I / (2.0f * (float)A1.H);
        const int t0 = fs_split(blockIdx.x, G, F.nd2, total, d);
        const int t1 = fs_split(blockIdx.x + 1, G, F.nd2, total, d);
        if (t1 > t0)
            dec_tiles<FMT, 1, SPW1, kFsWaves, 2, false, true, SH, true, true>(A1, S, act, red, t0,
                                                                              t1 - t0);
    }
    // Arrival, once this workgroup's activation rows have reached the
    // coherence point: the tile code stores them from wavefront 0 only (the
    // K-split partial sums meet there).
    uint64_t want = 0;
    if (tid == 0) want = fs_arrive(F.sync, blockIdx.x, G);
    if ((int)blockIdx.x >= F.nd2) return;

    // 3. down + combine for output columns 16 rb .. 16 rb + 15
    constexpr int D = dc_depth<FMT, NS2>();
    static_assert(D >= 2, "down+combine needs two weight buffers");
    const int rb = blockIdx.x;
    const int nrows = F.nrows, ngroups = (nrows + 15) / 16;
    // (written only after the barrier, when the gate/up part's LDS is dead)
    uint8_t *actL = reg;
    float *yl = reinterpret_cast<float *>(reg + (size_t)ngroups * NS2 * 4096);

    const int nmine = act.count > wv ? (act.count - wv + kFsWaves - 1) / kFsWaves : 0;
    const DcMeta meta = fs_meta<FMT, SH>(A2, S, act, wv, nmine);
    DcExpert<FMT> es[D];
    WFrag<FMT> wr[D][NS2];
    // the weights of this wavefront's first D experts (every one it has at
    // these sizes) are requested before the wait, so they arrive during it
    if (nmine > 0) {
#pragma unroll
        for (int dd = 0; dd < D; ++dd) {
            dc_state<FMT>(A2, meta, dd < nmine ? dd : nmine - 1, es[dd]);
            dc_load<FMT, NS2>(es[dd], rb, lane, wr[dd], dd < nmine);
        }
    }
    if (tid < nrows) spl[tid] = tid < n ? act.lsrt[tid] : tid;
    if (tid < n) wl[tid] = rw[tid];
    // wait for every workgroup's activation rows (bounded)
    if (tid == 0) fs_wait(F.sync, blockIdx.x, want);
    __syncthreads();
    // the activation rows into LDS (rows past the end repeat the last one)
    const uint16_t *actg = A2.src;
    const int ndma = ngroups * NS2 * 4;
    for (int dd = wv; dd < ndma; dd += kFsWaves) {
        const int g = dd / (NS2 * 4), s = (dd >> 2) % NS2, j = dd & 3;
        int row = 16 * g + m;
        row = row < nrows ? row : nrows - 1;
        lds_dma16_coherent(actg + (size_t)row * A2.K + s * 128 + 32 * c + 8 * j,
                           actL + (size_t)dd * 1024);
    }
    wait_vm<0>();
    __syncthreads();
    if (nmine > 0) {
        for (int i = 0; i < nmine; i += D) {
#pragma unroll
            for (int dd = 0; dd < D; ++dd) {
                if (i + dd < nmine) {
                    dc_expert<FMT, NS2>(A2, es[dd], wr[dd], actL, yl, spl, rb, m, c, nrows);
                    // the buffer just used takes the expert D further on
                    const int qn = i + dd + D;
                    if (qn < nmine) {
                        dc_state<FMT>(A2, meta, qn, es[dd]);
                        dc_load<FMT, NS2>(es[dd], rb, lane, wr[dd], true);
                    }
                }
            }
        }
    }
    __syncthreads();
    const int t = tid >> 4, col = tid & 15;
    if (t < F.T) {
        float acc = 0.0f;
        for (int j = 0; j < k; ++j) acc += wl[t * k + j] * yl[(t * k + j) * 16 + col];
        if (SH) acc += yl[(n + t) * 16 + col];
        F.out[(size_t)t * A2.H + 16 * rb + col] = (uint16_t)f32_to_bf16_bits(acc);
    }
}

static size_t fs_lds_bytes(int E, int n, int nrows, int ns2) {
    const size_t p1 = fs_phase1_bytes(E, n), p3 = fs_phase3_bytes(nrows, ns2);
    return kFsHead + (p1 > p3 ? p1 : p3);
}

template <int SPW1, int NS2, bool SH>
static int launch_small(hipStream_t s, const DecArgs &A1, const DecArgs &A2, const ShArgs &S,
                        const FsArgs &F) {
    auto kern = ffn_small_kernel<SPW1, NS2, SH>;
    const size_t lds = fs_lds_bytes(A1.E, F.T * A1.k, F.nrows, NS2);
    static bool attr = false;
    // LDS size of the last occupancy query (high half) and its answer (low
    // half), in one word so that calls from several host threads read a
    // consistent pair
    static std::atomic<uint64_t> occ{0};
    if (!attr) {
        if (int rc = check_hip(hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   (int)kFsMaxLds)))
            return rc;
        attr = true;
    }
    if (lds > kFsMaxLds) return MOE_EUNSUPPORTED;
    // every workgroup resident at once, or no launch
    uint64_t o = occ.load(std::memory_order_relaxed);
    if ((o >> 32) != lds) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kWave * kFsWaves, lds) !=
            hipSuccess || per_cu < 0)
            per_cu = 0;
        o = ((uint64_t)lds << 32) | (uint32_t)per_cu;
        occ.store(o, std::memory_order_relaxed);
    }
    if ((uint32_t)o < 1) return MOE_EUNSUPPORTED;
    const int G = num_cus();
    if (F.nd2 > G || G % kFsGroups) return MOE_EUNSUPPORTED;
    MOE_LAUNCH(K_DEC_SMALL, kern, dim3((unsigned)G), dim3(kWave * kFsWaves), lds, s, A1, A2, S, F);
    return check_launch();
}

// Whether the one-launch layer takes this batch (host check, no device work).
static bool small_eligible(int fmt, int T, int k, bool sh, int H, int I, int E) {
    if (fmt != MOE_W_MXFP4 || T < 1 || T > kFsWaves || k < 1 || E < 1 || E > kIdsMaxE) return false;
    if (k > E) return false;
    const int nrows = T * k + (sh ? T : 0);
    if (nrows > kFsMaxRows || H % 1024 || I % 128) return false;
    const int slabs1 = H / 128, ns2 = I / 128;
    if (slabs1 != 8 && slabs1 != 16 && slabs1 != 32) return false;
    return ns2 == 4 || ns2 == 6 || ns2 == 16;
}

template <bool SH>
static int ffn_small_fmt(const uint16_t *x, const float *logits, const moe_expert_w *experts,
                         const moe_expert_w *shared, int T, int k, int H, int I, int E,
                         int renorm, int32_t *topk_ids, float *topk_w, int32_t *offsets,
                         int32_t *sorted_pair, int32_t *pair_row, uint16_t *y, uint16_t *out,
                         uint16_t *act, uint64_t *sync, hipStream_t s) {
    const ShArgs S{shared, T, T * k};
    DecArgs a1{x, sorted_pair, offsets, experts, act, k, H, H, I, E, I / 16, 1, 0.0f, 0.0f};
    const DecArgs a2{act, sorted_pair, offsets, experts, y, k, I, H, I, E, 0, 1, 0.0f, 0.0f};
    const FsArgs F{logits, topk_ids, topk_w, pair_row, out, sync, T, renorm,
                   T * k + (SH ? T : 0), H / 16};
    const int slabs1 = H / 128, ns2 = I / 128;
#define MOE_FS(SPW1_, NS2_) \
    if (slabs1 == 8 * SPW1_ && ns2 == NS2_) return launch_small<SPW1_, NS2_, SH>(s, a1, a2, S, F)
    MOE_FS(1, 4);
    MOE_FS(2, 6);
    MOE_FS(4, 16);
    MOE_FS(2, 4);
    MOE_FS(4, 6);
#undef MOE_FS
    return MOE_EUNSUPPORTED;
}

int ffn_small_layer(const uint16_t *x, const float *logits, const moe_expert_w *experts,
                    const moe_expert_w *shared, int fmt, int T, int k, int H, int I, int E,
                    int renorm, int32_t *topk_ids, float *topk_w, int32_t *offsets,
                    int32_t *sorted_pair, int32_t *pair_row, uint16_t *y, uint16_t *out,
                    uint16_t *act, uint64_t *sync, hipStream_t s) {
    if (!small_eligible(fmt, T, k, shared != nullptr, H, I, E)) return MOE_EUNSUPPORTED;
    if (shared)
        return ffn_small_fmt<true>(x, logits, experts, shared, T, k, H, I, E, renorm, topk_ids,
                                   topk_w, offsets, sorted_pair, pair_row, y, out, act, sync, s);
    return ffn_small_fmt<false>(x, logits, experts, nullptr, T, k, H, I, E, renorm, topk_ids,
                                topk_w, offsets, sorted_pair, pair_row, y, out, act, sync, s);
}

}  // namespace moe
