// Prefill-shaped grouped SwiGLU expert FFN (tiled matrix-core GEMM).
#include "common.hpp"

namespace moe {

bool ffn_prefill_supported(int, int, int) { return false; }

int ffn_prefill(const uint16_t *, const int32_t *, const int32_t *, const moe_expert_w *, int, int,
                int, int, int, int, void *, int, uint16_t *, hipStream_t) {
    return MOE_EUNSUPPORTED;
}

}  // namespace moe
