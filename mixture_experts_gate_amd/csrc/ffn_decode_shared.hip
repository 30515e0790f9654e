// Weight-streaming expert FFN with the shared expert as one more expert of the
// routed launches (moe_expert_ffn_shared): the kernels of ffn_decode.hip with
// their shared-expert path switched on, instantiated in this translation unit.
#define MOE_DEC_SHARED_UNIT 1
#include "ffn_decode.hip"
