// GEMM instantiations for transA='N', transB='N' (A K-contiguous, B N-contiguous).
#include "gemm_kernel.h"

namespace tgemm {
hipError_t launch_gemm_nn(int cfg, int epi, const GemmParams& p, hipStream_t s) {
  return launch_gemm_layout<true, false>(cfg, epi, p, s);
}
}  // namespace tgemm
