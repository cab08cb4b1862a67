// Exact attention backward (placeholder until the MFMA kernels land).
#include "common.hpp"
#include "launch.hpp"

namespace bea {

size_t bwd_workspace_bytes(int n, int l_q, int h) {
  return (size_t)n * l_q * h * sizeof(float);
}

hipError_t launch_bwd(const void*, const void*, const void*, const void*,
                      const void*, const float*, void*, void*, void*,
                      const AttnShape&, void*, bool, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace bea
