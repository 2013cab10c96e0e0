// KV-block-major prefill attention (placeholder until the kernel lands).
#include "msa_device.h"

namespace msa {
size_t prefill_workspace_bytes(int32_t Nq, int32_t Hkv, int32_t k, int32_t num_pages) { return 256; }
hipError_t launch_attn_prefill(int, int, int, int, int, int, const int32_t*, const int32_t*, const int32_t*,
                               const int32_t*, const void*, const void*, const void*, int, const int32_t*,
                               const int32_t*, int, float, void*, float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace msa
