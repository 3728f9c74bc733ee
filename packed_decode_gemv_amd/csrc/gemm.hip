// Batched dequantise-and-multiply on MFMA (placeholder until the tile kernel lands).
#include "vbq_common.h"

namespace vbq {

hipError_t launch_gemm(const vbq_matrix& m, const uint16_t* x, int M, float* y, hipStream_t s) {
  (void)m; (void)x; (void)M; (void)y; (void)s;
  return hipErrorNotSupported;
}

}  // namespace vbq
