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
    "cache_move"};

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
int ffn_prefill(const uint16_t *x, const int32_t *sorted_pair, const int32_t *offsets,
                const moe_expert_w *experts, int fmt, int T, int k, int H, int I, int E, void *y,
                int y_is_fp32, void *ws, hipStream_t s);
bool ffn_prefill_supported(int fmt, int H, int I);
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

extern "C" int moe_expert_ffn(const uint16_t *x_bf16, const int32_t *sorted_pair,
                              const int32_t *offsets, const moe_expert_w *experts, int fmt, int T,
                              int k, int H, int I, int E, void *y, int y_is_fp32, void *ws,
                              size_t ws_bytes, void *stream) {
    // E <= 512: the weight-streaming kernels keep the set of active experts
    // as a 512-bit mask
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
        return ffn_prefill(x_bf16, sorted_pair, offsets, experts, fmt, T, k, H, I, E, y, y_is_fp32,
                           ws, s);
    return ffn_decode(x_bf16, sorted_pair, offsets, experts, fmt, T, k, H, I, E, y, y_is_fp32,
                      act, s);
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
    // the tiled kernels take the shared expert as its own call
    if (use_prefill(n, E, fmt, H, I)) return MOE_EUNSUPPORTED;
    return ffn_decode_shared(x_bf16, sorted_pair, offsets, experts, shared, fmt, T, k, H, I, E,
                             y, y_is_fp32, reinterpret_cast<uint16_t *>(ws),
                             (hipStream_t)stream);
}
