// Router kernel: one wavefront per token (see route_dev.hpp).
#include "route_dev.hpp"

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg,
    const float *__restrict__ logits_in, float *__restrict__ logits_out, int T, int H, int E,
    int k, int renormalize, int32_t *__restrict__ topk_ids, float *__restrict__ topk_w) {
    const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (t >= T) return;
    route_token<VPL>(t, x, wg, logits_in, logits_out, H, E, k, renormalize, topk_ids, topk_w);
}

}  // namespace moe


using namespace moe;

extern "C" int moe_route(const uint16_t *x_bf16, const uint16_t *wg_bf16, const float *logits_in,
                         float *logits_out, int T, int H, int E, int k, int renormalize,
                         int32_t *topk_ids, float *topk_w, void *stream) {
    if (T < 0 || E < 1 || E > 1024 || k < 1 || k > E || k > kWave) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!topk_ids || !topk_w) return MOE_EINVAL;
    if (!logits_in) {
        if (!x_bf16 || !wg_bf16 || H < 8 || H % 8) return MOE_EINVAL;
    }
    hipStream_t s = (hipStream_t)stream;
    const int waves_per_block = 4;
    dim3 grid((T + waves_per_block - 1) / waves_per_block), block(kWave * waves_per_block);
#define MOE_ROUTE_LAUNCH(VPL)                                                                 \
    MOE_LAUNCH(K_ROUTE, route_kernel<VPL>, grid, block, 0, s, x_bf16, wg_bf16,       \
                                 logits_in, logits_out, T, H, E, k, renormalize, topk_ids,    \
                                 topk_w)
    if (E <= 64) MOE_ROUTE_LAUNCH(1);
    else if (E <= 128) MOE_ROUTE_LAUNCH(2);
    else if (E <= 256) MOE_ROUTE_LAUNCH(4);
    else if (E <= 512) MOE_ROUTE_LAUNCH(8);
    else MOE_ROUTE_LAUNCH(16);
#undef MOE_ROUTE_LAUNCH
    return check_launch();
}
