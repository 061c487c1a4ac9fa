// GEMM instantiations for transA='T', transB='T' (A M-contiguous, B K-contiguous).
#include "gemm_kernel.h"

namespace tgemm {
hipError_t launch_gemm_tt(int cfg, int epi, const GemmParams& p, hipStream_t s) {
  return launch_gemm_layout<false, true>(cfg, epi, p, s);
}
}  // namespace tgemm
