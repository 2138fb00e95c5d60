// Fused LM-head forward/backward (placeholder until the MFMA kernels land).
#include <hip/hip_runtime.h>

#include "../../include/rlk.h"

extern "C" {

size_t rlk_logprob_fused_linear_workspace_size(int64_t, int64_t, int64_t, float) { return 0; }

rlk_status rlk_logprob_fused_linear(const void*, const void*, int64_t, int64_t, int64_t, int64_t,
                                    int64_t, const int64_t*, float, float, int32_t, float*, float*,
                                    float*, int32_t*, uint8_t*, void*, size_t, void*) {
  return RLK_EUNSUPPORTED;
}

size_t rlk_logprob_fused_linear_bwd_workspace_size(int64_t, int64_t, int64_t, float) { return 0; }

rlk_status rlk_logprob_fused_linear_bwd(const void*, const void*, int64_t, int64_t, int64_t,
                                        int64_t, int64_t, const int64_t*, const float*,
                                        const float*, const float*, float, float, int32_t, void*,
                                        float*, void*, size_t, void*) {
  return RLK_EUNSUPPORTED;
}

}  // extern "C"
