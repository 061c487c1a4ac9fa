// GEMM instantiations for transA='N', transB='T' (A K-contiguous, B K-contiguous).
#include "gemm_kernel.h"

namespace tgemm {
hipError_t launch_gemm_nt(int cfg, int epi, const GemmParams& p, hipStream_t s) {
  return launch_gemm_layout<true, true>(cfg, epi, p, s);
}
}  // namespace tgemm
