// Index-gather latent-attention decode for gfx950 (placeholder launcher; the
// kernel is not built yet and the launcher reports hipErrorNotSupported).
#include <hip/hip_runtime.h>

#include "mla.h"

namespace pkv {

int mla_workspace_bytes(int32_t batch, int32_t num_qo_heads, int32_t d_qk, int32_t d_v,
                        int32_t topk, size_t* bytes, std::string* err) {
  if (batch < 0 || topk < 0) { *err = "batch and topk must be >= 0"; return 1; }
  if (d_qk != kMlaDqk || d_v != kMlaDv) {
    *err = "expected d_qk=576 and d_v=512";
    return 2;
  }
  if (num_qo_heads <= 0 || num_qo_heads % 16 != 0 || num_qo_heads > kMlaMaxHeads) {
    *err = "num_qo_heads must be a multiple of 16 in [16, 128]";
    return 2;
  }
  *bytes = 0;
  return 0;
}

hipError_t launch_gather_mla(const uint16_t*, const uint16_t*, int64_t, const int32_t*, int32_t,
                             int32_t, int32_t, float, void*, uint16_t*, float*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace pkv
