// GEMM instantiations for transA='T', transB='N' (A M-contiguous, B N-contiguous).
#include "gemm_kernel.h"

namespace tgemm {
hipError_t launch_gemm_tn(int cfg, int epi, const GemmParams& p, hipStream_t s) {
  return launch_gemm_layout<false, false>(cfg, epi, p, s);
}
}  // namespace tgemm
