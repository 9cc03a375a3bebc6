// Prefill-shaped projection (long per-request segments): MFMA-bound tiled GEMM.
#include "device_common.h"
#include "internal.h"

namespace lorapool {

hipError_t launch_prefill(const lora_pool *, const Plan &, const Ws &, const void *, const void *, const int32_t *,
                          const float *, void *, hipStream_t, hipEvent_t) {
    return hipErrorNotSupported;
}

}  // namespace lorapool
