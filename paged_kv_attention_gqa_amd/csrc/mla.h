// Index-gather latent-attention decode (bf16 latent rows of 576 dims whose
// first 512 dims are the values). Implemented in mla.hip.
#ifndef PKV_MLA_H_
#define PKV_MLA_H_

#include <hip/hip_runtime_api.h>

#include <cstddef>
#include <cstdint>
#include <string>

namespace pkv {

constexpr int kMlaDqk = 576;
constexpr int kMlaDv = 512;
constexpr int kMlaMaxHeads = 128;
// FP8 token: 512 e4m3 values, 4 fp32 scales (one per 128 values), 64 bf16 values.
constexpr int kMlaFp8TokenBytes = 656;
// The list is cut into pieces so that about this many workgroups run; fixed so
// that the workspace size depends on the shape only.
constexpr int kMlaPlanCus = 256;

// Device scratch held by the library for pkv_gather_mla_noalloc: one array of
// this many bytes per GPU, alive until the process ends (48 MiB: the fp32
// partials of a batch of 32 rows x 128 heads cut into 4 pieces take 33.6 MB).
constexpr size_t kMlaScratchBytes = size_t(48) << 20;

// Address of this library's device scratch on the current device, looked up
// (hipGetSymbolAddress) on the first call made with that device current.
hipError_t mla_scratch(void** ptr);

// Checks the gather shape; returns 0 and the workspace size, or a pkv_status
// code with a message.
int mla_workspace_bytes(int32_t batch, int32_t num_qo_heads, int32_t d_qk, int32_t d_v,
                        int32_t topk, size_t* bytes, std::string* err);

// kv_pool: bf16 [pool_tokens, 576], or [pool_tokens, 656] bytes when fp8_pool.
// attn_sink: fp32 [num_qo_heads] or NULL; topk_length: int32 [batch] or NULL.
hipError_t launch_gather_mla(const uint16_t* q, const void* kv_pool, bool fp8_pool,
                             int64_t pool_tokens, const int32_t* indices, int32_t topk,
                             int32_t batch, int32_t num_qo_heads, float sm_scale,
                             const float* attn_sink, const int32_t* topk_length, void* workspace,
                             uint16_t* out, float* lse, hipStream_t stream);

}  // namespace pkv

#endif  // PKV_MLA_H_
