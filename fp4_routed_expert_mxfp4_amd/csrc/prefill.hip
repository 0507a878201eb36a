// Prefill expert FFN on gfx950 block-scaled MFMA (placeholder until the MFMA
// kernels land: reports that no kernel exists for the call).
#include "common.cuh"
#include "kernels.h"

namespace moe {

size_t prefill_workspace_bytes(int T, int k, int H, int I) {
  (void)T; (void)k; (void)H; (void)I;
  return 256;
}

hipError_t launch_prefill(const uint16_t*, int, int, int, const ExpertStore&, const int32_t*, const int32_t*,
                          const int32_t*, float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moe
