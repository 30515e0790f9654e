// C-ABI glue: error text, options, workspace sizing and the expert-FFN
// dispatcher (decode-shaped weight streaming vs prefill-shaped tiled GEMM).
#include <atomic>
#include <mutex>
#include <vector>

#include "common.hpp"

namespace moe {

static thread_local int g_last_hip_error = 0;
static std::atomic<int> g_ffn_path{0};

void set_last_hip_error(hipError_t e) { g_last_hip_error = (int)e; }
int ffn_path_option() { return g_ffn_path.load(); }

// Decode tile-split weights, one byte each in units of 1/256: stage 1 slot,
// stage 1 position, stage 2 slot, stage 2 position (low byte first).
// tiled kernels: weight tiles per workgroup, stage 1 in the low byte, stage 2 next
constexpr int kPreGroupDefault = 1 | (2 << 8);
static std::atomic<int> g_pre_group{kPreGroupDefault};
int pre_group(int stage) {
    const int v = g_pre_group.load(std::memory_order_relaxed);
    const int g = stage == 1 ? (v & 0xFF) : ((v >> 8) & 0xFF);
    return g < 1 ? 1 : g;
}

// measured on the decode layer at T = 8..64 and the large sparse layer at
// T = 64 (graph-replayed steps): stage 1 96/256 by slot and none by position
// within a slot (68.3 against 69.9 us per T=64 step with 64/256 and 38/256),
// stage 2 38/256 and 23/256
constexpr int kDecSplitDefault = 96 | (0 << 8) | (38 << 16) | (23 << 24);
static std::atomic<int> g_dec_split{kDecSplitDefault};
void dec_split_weights(int stage, float *w_slot, float *w_pos) {
    const unsigned v = (unsigned)g_dec_split.load(std::memory_order_relaxed);
    const int sh = stage == 1 ? 0 : 16;
    *w_slot = (float)((v >> sh) & 0xFF) / 256.0f;
    *w_pos = (float)((v >> (sh + 8)) & 0xFF) / 256.0f;
}

// ---------------------------------------------------------------- timing --
// Optional per-kernel launch timing: each launch is made with
// hipExtLaunchKernel and two events that take the dispatch's own start and end
// times on its stream; moe_timing_query sums the elapsed times.
static std::atomic<bool> g_timing{false};
static std::mutex g_tmu;
struct TimingRec {
    int kid;
    hipEvent_t a, b;
};
static std::vector<TimingRec> g_recs;        // launches awaiting a query
static std::vector<hipEvent_t> g_evpool;
static long long g_launches[K_COUNT];
static double g_ms[K_COUNT];

static const char *const g_kernel_names[K_COUNT] = {
    "route", "permute_small", "permute_rank", "permute_scan", "permute_scatter", "permute_empty",
    "ffn_decode_gate_up", "ffn_decode_down", "ffn_prefill_gate_up", "ffn_prefill_down",
    "combine", "cache_table", "pack_mxfp4", "route_permute", "ffn_prefill_split",
    "cache_move", "micro_read", "micro_mfma", "scatter_rows", "layer_fused"};

static hipEvent_t pool_event() {
    if (!g_evpool.empty()) {
        hipEvent_t e = g_evpool.back();
        g_evpool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    (void)hipEventCreate(&e);
    return e;
}

bool timing_enabled() { return g_timing.load(std::memory_order_relaxed); }

bool timing_begin(int kid, hipEvent_t *start, hipEvent_t *stop) {
    std::lock_guard<std::mutex> lk(g_tmu);
    TimingRec r{kid, pool_event(), pool_event()};
    if (!r.a || !r.b) {
        if (r.a) g_evpool.push_back(r.a);
        if (r.b) g_evpool.push_back(r.b);
        return false;
    }
    g_recs.push_back(r);
    *start = r.a;
    *stop = r.b;
    return true;
}

static void timing_drain() {
    for (TimingRec &r : g_recs) {
        float ms = 0.0f;
        if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
            g_ms[r.kid] += ms;
            g_launches[r.kid] += 1;
        }
        g_evpool.push_back(r.a);
        g_evpool.push_back(r.b);
    }
    g_recs.clear();
}

size_t permute_ws_bytes(long n, int E);
int ffn_decode(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
               const moe_expert_w *experts, int fmt, int T, int k, int H, int I, int E, void *y,
               int y_is_fp32, uint16_t *act, hipStream_t s);
int ffn_decode_shared(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
                      const moe_expert_w *experts, const moe_expert_w *shared, int fmt, int T,
                      int k, int H, int I, int E, void *y, int y_is_fp32, uint16_t *act,
                      hipStream_t s);
int ffn_decode_comb(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
                    const moe_expert_w *experts, int fmt, const float *topk_w, int T, int k,
                    int H, int I, int E, uint16_t *y, uint16_t *out, uint16_t *act, hipStream_t s);
int ffn_decode_comb_shared(const uint16_t *x, const int32_t *sorted_pair,
                           const int32_t *offsets, const moe_expert_w *experts,
                           const moe_expert_w *shared, int fmt, const float *topk_w, int T,
                           int k, int H, int I, int E, uint16_t *y, uint16_t *out, uint16_t *act,
                           hipStream_t s);
int ffn_decode_ids(const uint16_t *x, const int32_t *ids, const moe_expert_w *experts, int fmt,
                   int T, int k, int H, int I, int E, void *y, int y_is_fp32, int32_t *offsets,
                   int32_t *sorted_pair, int32_t *pair_row, uint16_t *act, hipStream_t s);
int ffn_decode_ids_shared(const uint16_t *x, const int32_t *ids, const moe_expert_w *experts,
                          const moe_expert_w *shared, int fmt, int T, int k, int H, int I, int E,
                          void *y, int y_is_fp32, int32_t *offsets, int32_t *sorted_pair,
                          int32_t *pair_row, uint16_t *act, hipStream_t s);
int ffn_decode_ids_comb(const uint16_t *x, const int32_t *ids, const moe_expert_w *experts,
                        int fmt, const float *topk_w, int T, int k, int H, int I, int E,
                        uint16_t *y, uint16_t *out, int32_t *offsets, int32_t *sorted_pair,
                        int32_t *pair_row, uint16_t *act, hipStream_t s);
int ffn_decode_ids_comb_shared(const uint16_t *x, const int32_t *ids,
                               const moe_expert_w *experts, const moe_expert_w *shared, int fmt,
                               const float *topk_w, int T, int k, int H, int I, int E,
                               uint16_t *y, uint16_t *out, int32_t *offsets,
                               int32_t *sorted_pair, int32_t *pair_row, uint16_t *act,
                               hipStream_t s);
int ffn_prefill(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
                const moe_expert_w *experts, const moe_expert_w *shared, int fmt, int T, int k,
                int H, int I, int E, void *y, int y_is_fp32, void *ws, hipStream_t s);
bool ffn_prefill_supported(int fmt, int H, int I);
int ffn_small_layer(const uint16_t *x, const float *logits, const moe_expert_w *experts,
                    const moe_expert_w *shared, int fmt, int T, int k, int H, int I, int E,
                    int renorm, int32_t *topk_ids, float *topk_w, int32_t *offsets,
                    int32_t *sorted_pair, int32_t *pair_row, uint16_t *y, uint16_t *out,
                    uint16_t *act, uint64_t *sync, hipStream_t s);
size_t prefill_ws_bytes(long n_pairs, long T, int H, int I, int E);

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Decode kernels keep the bf16 activation [n_pairs][I]; the tiled kernels the
// two-term FP8 activation and token rows. Either may run, so the larger.
size_t ffn_ws_bytes(long n_pairs, long T, int H, int I, int E) {
    const size_t dec = align256((size_t)n_pairs * I * 2);
    const size_t pre = prefill_ws_bytes(n_pairs, T, H, I, E);
    return (dec > pre ? dec : pre) + 256;
}

// Decode kernels stream each touched expert once; prefill kernels tile the
// contraction for the matrix cores. The tiled path needs many rows per expert
// (48 on average) and enough 128-row x 128-column tiles to give every compute
// unit at least one (a single shared expert over a few dozen tokens has 16).
static bool use_prefill(long n_pairs, int E, int fmt, int H, int I) {
    const int opt = g_ffn_path.load();
    if (opt == 1) return false;
    if (opt == 2) return ffn_prefill_supported(fmt, H, I);
    return ffn_prefill_supported(fmt, H, I) && n_pairs >= 48L * E &&
           (n_pairs / 128) * (I / 128) >= 256;
}

}  // namespace moe

using namespace moe;

extern "C" const char *moe_strerror(int err) {
    switch (err) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_ENOMEM: return "not enough memory or cache slots";
        case MOE_EHIP: return "HIP runtime error";
        case MOE_EUNSUPPORTED: return "unsupported request";
        case MOE_EBUSY: return "resource busy";
        default: return "unknown error";
    }
}

extern "C" int moe_last_hip_error(void) { return g_last_hip_error; }

extern "C" int moe_set_option(int option, int value) {
    if (option == MOE_OPT_FFN_PATH) {
        if (value < 0 || value > 2) return MOE_EINVAL;
        g_ffn_path.store(value);
        return MOE_OK;
    }
    if (option == MOE_OPT_PRE_GROUP) {
        if (value == -1) value = kPreGroupDefault;
        if (value < 0 || (value & 0xFF) < 1 || (value & 0xFF) > 16 || ((value >> 8) & 0xFF) < 1 ||
            ((value >> 8) & 0xFF) > 16 || (value >> 16))
            return MOE_EINVAL;
        g_pre_group.store(value);
        return MOE_OK;
    }
    if (option == MOE_OPT_CACHE_FAULT) return cache_set_fault(value);
    if (option == MOE_OPT_CACHE_DELAY_US) return cache_set_delay(value);
    if (option == MOE_OPT_CACHE_THROTTLE_MBS) return cache_set_throttle(value);
    if (option == MOE_OPT_DEC_SPLIT) {
        if (value == -1) value = kDecSplitDefault;
        // every byte below 128: each weight stays under one half
        if (value < 0 || (value & 0x80808080)) return MOE_EINVAL;
        g_dec_split.store(value);
        return MOE_OK;
    }
    if (option == MOE_OPT_TIMING) {
        if (value < 0 || value > 1) return MOE_EINVAL;
        std::lock_guard<std::mutex> lk(g_tmu);
        timing_drain();
        for (int i = 0; i < K_COUNT; ++i) {
            g_launches[i] = 0;
            g_ms[i] = 0.0;
        }
        g_timing.store(value == 1);
        return MOE_OK;
    }
    return MOE_EINVAL;
}

extern "C" int moe_get_option(int option) {
    if (option == MOE_OPT_FFN_PATH) return g_ffn_path.load();
    if (option == MOE_OPT_TIMING) return g_timing.load() ? 1 : 0;
    if (option == MOE_OPT_DEC_SPLIT) return g_dec_split.load();
    if (option == MOE_OPT_PRE_GROUP) return g_pre_group.load();
    if (option == MOE_OPT_CACHE_FAULT) return cache_get_fault();
    if (option == MOE_OPT_CACHE_DELAY_US) return cache_get_delay();
    if (option == MOE_OPT_CACHE_THROTTLE_MBS) return cache_get_throttle();
    return MOE_EINVAL;
}

extern "C" const char *moe_kernel_name(int kernel_id) {
    if (kernel_id < 0 || kernel_id >= K_COUNT) return nullptr;
    return g_kernel_names[kernel_id];
}

extern "C" int moe_timing_query(int kernel_id, long long *launches, double *total_ms) {
    if (kernel_id < 0 || kernel_id >= K_COUNT) return MOE_EINVAL;
    std::lock_guard<std::mutex> lk(g_tmu);
    timing_drain();
    if (launches) *launches = g_launches[kernel_id];
    if (total_ms) *total_ms = g_ms[kernel_id];
    return MOE_OK;
}

extern "C" int moe_workspace_size(int T, int k, int H, int I, int E, size_t *permute_bytes,
                                  size_t *ffn_bytes) {
    if (T < 0 || k < 1 || E < 1 || H < 32 || I < 32) return MOE_EINVAL;
    const long n = (long)T * k;
    if (permute_bytes) *permute_bytes = permute_ws_bytes(n, E);
    if (ffn_bytes) *ffn_bytes = ffn_ws_bytes(n, T, H, I, E);
    return MOE_OK;
}

namespace moe {
// The expert FFN behind moe_expert_ffn (and its variant without a caller
// workspace): argument checks, then the weight-streaming or tiled kernels.
int expert_ffn_call(const uint16_t *x_bf16, const int32_t *sorted_pair, const int32_t *offsets,
                    const moe_expert_w *experts, int fmt, int T, int k, int H, int I, int E,
                    void *y, int y_is_fp32, void *ws, size_t ws_bytes, void *stream) {
    // E <= 512: the weight-streaming kernels scan the active experts in
    // eight groups of 64
    if (T < 0 || k < 1 || E < 1 || E > 512 || H < 32 || I < 32 || H % 32 || I % 32)
        return MOE_EINVAL;
    if (fmt != MOE_W_MXFP4 && fmt != MOE_W_BF16 && fmt != MOE_W_NVFP4 && fmt != MOE_W_FP8)
        return MOE_EINVAL;
    if (fmt != MOE_W_BF16 && (H % 128 || I % 128)) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!x_bf16 || !sorted_pair || !offsets || !experts || !y || !ws) return MOE_EINVAL;
    const long n = (long)T * k;
    if (n > 0x7FFFFFFFL) return MOE_EINVAL;
    if (ws_bytes < ffn_ws_bytes(n, T, H, I, E)) return MOE_EINVAL;
    uint16_t *act = reinterpret_cast<uint16_t *>(ws);
    hipStream_t s = (hipStream_t)stream;
    if (use_prefill(n, E, fmt, H, I))
        return ffn_prefill(x_bf16, sorted_pair, offsets, experts, nullptr, fmt, T, k, H, I, E, y,
                           y_is_fp32, ws, s);
    return ffn_decode(x_bf16, sorted_pair, offsets, experts, fmt, T, k, H, I, E, y, y_is_fp32,
                      act, s);
}
}  // namespace moe

extern "C" int moe_expert_ffn(const uint16_t *x_bf16, const int32_t *sorted_pair,
                              const int32_t *offsets, const moe_expert_w *experts, int fmt, int T,
                              int k, int H, int I, int E, void *y, int y_is_fp32, void *ws,
                              size_t ws_bytes, void *stream) {
    return expert_ffn_call(x_bf16, sorted_pair, offsets, experts, fmt, T, k, H, I, E, y,
                           y_is_fp32, ws, ws_bytes, stream);
}

extern "C" int moe_expert_ffn_shared(const uint16_t *x_bf16, const int32_t *sorted_pair,
                                     const int32_t *offsets, const moe_expert_w *experts,
                                     const moe_expert_w *shared, int fmt, int T, int k, int H,
                                     int I, int E, void *y, int y_is_fp32, void *ws,
                                     size_t ws_bytes, void *stream) {
    if (T < 0 || k < 1 || E < 1 || E > 512 || H < 32 || I < 32 || H % 32 || I % 32)
        return MOE_EINVAL;
    if (fmt != MOE_W_MXFP4 && fmt != MOE_W_BF16 && fmt != MOE_W_NVFP4 && fmt != MOE_W_FP8)
        return MOE_EINVAL;
    if (fmt != MOE_W_BF16 && (H % 128 || I % 128)) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!x_bf16 || !sorted_pair || !offsets || !experts || !shared || !y || !ws) return MOE_EINVAL;
    const long n = (long)T * k;
    if ((long)T * (k + 1) > 0x7FFFFFFFL) return MOE_EINVAL;
    // the activation holds the routed rows and then the shared expert's T rows
    if (ws_bytes < ffn_ws_bytes((long)T * (k + 1), T, H, I, E)) return MOE_EINVAL;
    // the shared expert is one more expert of the launches on either path
    if (use_prefill(n, E, fmt, H, I))
        return ffn_prefill(x_bf16, sorted_pair, offsets, experts, shared, fmt, T, k, H, I, E, y,
                           y_is_fp32, ws, (hipStream_t)stream);
    return ffn_decode_shared(x_bf16, sorted_pair, offsets, experts, shared, fmt, T, k, H, I, E,
                             y, y_is_fp32, reinterpret_cast<uint16_t *>(ws),
                             (hipStream_t)stream);
}

extern "C" int moe_expert_ffn_combine(const uint16_t *x_bf16, const int32_t *sorted_pair,
                                      const int32_t *offsets, const moe_expert_w *experts,
                                      const moe_expert_w *shared, int fmt, int T, int k, int H,
                                      int I, int E, const float *topk_w, uint16_t *y_bf16,
                                      uint16_t *out_bf16, void *ws, size_t ws_bytes,
                                      void *stream) {
    if (T < 0 || k < 1 || E < 1 || E > 512 || H < 32 || I < 32 || H % 32 || I % 32)
        return MOE_EINVAL;
    if (fmt != MOE_W_MXFP4 && fmt != MOE_W_BF16 && fmt != MOE_W_NVFP4 && fmt != MOE_W_FP8)
        return MOE_EINVAL;
    if (fmt != MOE_W_BF16 && (H % 128 || I % 128)) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!x_bf16 || !sorted_pair || !offsets || !experts || !topk_w || !y_bf16 || !out_bf16 || !ws)
        return MOE_EINVAL;
    const long n = (long)T * k;
    const long rows = n + (shared ? T : 0);
    if (rows > 0x7FFFFFFFL) return MOE_EINVAL;
    if (ws_bytes < ffn_ws_bytes(rows, T, H, I, E)) return MOE_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (!use_prefill(n, E, fmt, H, I)) {
        uint16_t *act = reinterpret_cast<uint16_t *>(ws);
        const int rc = shared ? ffn_decode_comb_shared(x_bf16, sorted_pair, offsets, experts,
                                                       shared, fmt, topk_w, T, k, H, I, E,
                                                       y_bf16, out_bf16, act, s)
                              : ffn_decode_comb(x_bf16, sorted_pair, offsets, experts, fmt,
                                                topk_w, T, k, H, I, E, y_bf16, out_bf16, act, s);
        if (rc != MOE_EUNSUPPORTED) return rc;
    }
    // the two calls
    const int rc = shared ? moe_expert_ffn_shared(x_bf16, sorted_pair, offsets, experts, shared,
                                                  fmt, T, k, H, I, E, y_bf16, 0, ws, ws_bytes,
                                                  stream)
                          : expert_ffn_call(x_bf16, sorted_pair, offsets, experts, fmt, T, k, H,
                                            I, E, y_bf16, 0, ws, ws_bytes, stream);
    if (rc) return rc;
    return moe_combine(y_bf16, 0, topk_w, shared ? y_bf16 + (size_t)n * H : nullptr, T, k, H,
                       out_bf16, stream);
}

extern "C" int moe_layer_fused(const uint16_t *x_bf16, const float *logits,
                               const moe_expert_w *experts, const moe_expert_w *shared, int fmt,
                               int T, int k, int H, int I, int E, int renormalize,
                               int32_t *topk_ids, float *topk_w, int32_t *offsets,
                               int32_t *sorted_pair, int32_t *pair_row, uint16_t *y_bf16,
                               uint16_t *out_bf16, void *ws, size_t ws_bytes, void *sync,
                               void *stream) {
    if (T < 1 || k < 1 || E < 1 || k > E || H < 128 || I < 128 || H % 128 || I % 128)
        return MOE_EINVAL;
    if (fmt != MOE_W_MXFP4 && fmt != MOE_W_BF16 && fmt != MOE_W_NVFP4 && fmt != MOE_W_FP8)
        return MOE_EINVAL;
    if (!x_bf16 || !logits || !experts || !topk_ids || !topk_w || !offsets || !sorted_pair ||
        !pair_row || !y_bf16 || !out_bf16 || !ws || !sync || (uintptr_t)sync % 8)
        return MOE_EINVAL;
    const long rows = (long)T * k + (shared ? T : 0);
    if (rows > 0x7FFFFFFFL) return MOE_EINVAL;
    if (ws_bytes < ffn_ws_bytes(rows, T, H, I, E)) return MOE_EINVAL;
    return ffn_small_layer(x_bf16, logits, experts, shared, fmt, T, k, H, I, E, renormalize,
                           topk_ids, topk_w, offsets, sorted_pair, pair_row, y_bf16, out_bf16,
                           reinterpret_cast<uint16_t *>(ws), reinterpret_cast<uint64_t *>(sync),
                           (hipStream_t)stream);
}

extern "C" int moe_permute_ffn_combine(const uint16_t *x_bf16, const int32_t *topk_ids,
                                       const float *topk_w, const moe_expert_w *experts,
                                       const moe_expert_w *shared, int fmt, int T, int k, int H,
                                       int I, int E, int32_t *offsets, int32_t *sorted_pair,
                                       int32_t *pair_row, uint16_t *y_bf16, uint16_t *out_bf16,
                                       void *ws, size_t ws_bytes, void *stream) {
    if (T < 0 || k < 1 || E < 1 || E > 512 || H < 32 || I < 32 || H % 32 || I % 32)
        return MOE_EINVAL;
    if (fmt != MOE_W_MXFP4 && fmt != MOE_W_BF16 && fmt != MOE_W_NVFP4 && fmt != MOE_W_FP8)
        return MOE_EINVAL;
    if (fmt != MOE_W_BF16 && (H % 128 || I % 128)) return MOE_EINVAL;
    if (!offsets) return MOE_EINVAL;
    if (T > 0 && (!x_bf16 || !topk_ids || !topk_w || !experts || !sorted_pair || !pair_row ||
                  !y_bf16 || !out_bf16 || !ws))
        return MOE_EINVAL;
    const long n = (long)T * k;
    const long rows = n + (shared ? T : 0);
    if (rows > 0x7FFFFFFFL) return MOE_EINVAL;
    if (T > 0 && ws_bytes < ffn_ws_bytes(rows, T, H, I, E)) return MOE_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    // the permutation inside the gate/up launch (weight-streaming kernels):
    // then the down projection and the combine in one launch (at most 15
    // rows), or the down launch and the combine
    if (T > 0 && !use_prefill(n, E, fmt, H, I)) {
        uint16_t *act = reinterpret_cast<uint16_t *>(ws);
        int rc = shared ? ffn_decode_ids_comb_shared(x_bf16, topk_ids, experts, shared, fmt,
                                                     topk_w, T, k, H, I, E, y_bf16, out_bf16,
                                                     offsets, sorted_pair, pair_row, act, s)
                        : ffn_decode_ids_comb(x_bf16, topk_ids, experts, fmt, topk_w, T, k, H, I,
                                              E, y_bf16, out_bf16, offsets, sorted_pair,
                                              pair_row, act, s);
        if (rc != MOE_EUNSUPPORTED) return rc;
        rc = shared ? ffn_decode_ids_shared(x_bf16, topk_ids, experts, shared, fmt, T, k, H, I,
                                            E, y_bf16, 0, offsets, sorted_pair, pair_row, act, s)
                    : ffn_decode_ids(x_bf16, topk_ids, experts, fmt, T, k, H, I, E, y_bf16, 0,
                                     offsets, sorted_pair, pair_row, act, s);
        if (rc != MOE_EUNSUPPORTED) {
            if (rc) return rc;
            return moe_combine(y_bf16, 0, topk_w, shared ? y_bf16 + (size_t)n * H : nullptr, T,
                               k, H, out_bf16, stream);
        }
    }
    // the two calls (the permutation's workspace, when it needs one, is the
    // FFN's: the stream runs the permutation before the FFN uses it)
    int rc = moe_permute(topk_ids, T, k, E, offsets, sorted_pair, pair_row, ws, ws_bytes, stream);
    if (rc) return rc;
    return moe_expert_ffn_combine(x_bf16, sorted_pair, offsets, experts, shared, fmt, T, k, H, I,
                                  E, topk_w, y_bf16, out_bf16, ws, ws_bytes, stream);
}
