// moe_expert_ffn for callers that cannot allocate device memory (code under
// graph capture, tight serving loops, harnesses that forbid allocation): the
// FFN's workspace is a fixed device array of this library instead of a
// caller buffer. The kernels are those of moe_expert_ffn; they receive the
// array's device address as their workspace argument.
#include <mutex>

#include "common.hpp"

namespace moe {

int expert_ffn_call(const uint16_t *x_bf16, const int32_t *sorted_pair, const int32_t *offsets,
                    const moe_expert_w *experts, int fmt, int T, int k, int H, int I, int E,
                    void *y, int y_is_fp32, void *ws, size_t ws_bytes, void *stream);
size_t ffn_ws_bytes(long n_pairs, long T, int H, int I, int E);

constexpr size_t kScratchBytes = MOE_FFN_NOALLOC_MAX_WS;

// One copy per device, allocated with the code object when the library's
// kernels are loaded on that device, held until the process ends. In host
// code this name is only a handle for the symbol lookup below: the device
// address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array, looked up on the
// first call made on that device and kept.
static int scratch_address(void **out) {
    int dev = 0;
    int rc = check_hip(hipGetDevice(&dev));
    if (rc) return rc;
    if (dev < 0 || dev >= kMaxDevices) return MOE_EUNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        rc = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (rc) return rc;
        if (!p) return MOE_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_expert_ffn_noalloc(const uint16_t *x_bf16, const int32_t *sorted_pair,
                                      const int32_t *offsets, const moe_expert_w *experts,
                                      int fmt, int T, int k, int H, int I, int E, void *y,
                                      int y_is_fp32, void *stream) {
    // sizes the library cannot serve from the array are refused before any
    // device work (argument errors are reported as by moe_expert_ffn)
    if (T > 0 && k >= 1 && E >= 1 && H >= 32 && I >= 32 && (long)T * k <= 0x7FFFFFFFL &&
        ffn_ws_bytes((long)T * k, T, H, I, E) > kScratchBytes)
        return MOE_ENOMEM;
    void *ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc) return rc;
    return expert_ffn_call(x_bf16, sorted_pair, offsets, experts, fmt, T, k, H, I, E, y,
                           y_is_fp32, ws, kScratchBytes, stream);
}
