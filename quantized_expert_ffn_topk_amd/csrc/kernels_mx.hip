// kernels_mx.hip -- MXFP4 expert FFNs (E2M1 weights, E8M0 scales per 32,
// bf16 activations) for gfx950.
#include "device_common.h"
#include "host_common.h"

namespace moe {

moe_status mx_ffn_enqueue(moe_ctx *, const void *, int, const moe_layer_weights *,
                          const void *const *, const int32_t *, const float *, void *, hipStream_t)
{
    return fail(MOE_E_UNSUPPORTED, "mxfp4 expert path not available");
}

}  // namespace moe
