// Sparse MQA attention backward (placeholder until the kernels land).
#include "common.hpp"
#include "launch.hpp"

namespace dsa {

size_t attn_bwd_workspace_bytes(int64_t nq, int h) {
  return static_cast<size_t>(nq > 0 ? nq : 0) * static_cast<size_t>(h > 0 ? h : 0) * sizeof(float);
}

hipError_t launch_sparse_attn_bwd(const void*, const void*, int64_t, const void*, int64_t,
                                  const int32_t*, int, const void*, int, const float*, const void*,
                                  float*, float*, float*, int64_t, int64_t, int, int, int, float,
                                  void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace dsa
