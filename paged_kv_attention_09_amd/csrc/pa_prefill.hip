// Chunked-prefill kernel (placeholder until the MFMA kernel lands).
#include "pa_kernels.hpp"

namespace pa {

hipError_t launch_prefill(const PrefillArgs &a, int head_dim, int group, hipStream_t stream) {
  (void)a; (void)head_dim; (void)group; (void)stream;
  return hipErrorInvalidValue;
}

}  // namespace pa
