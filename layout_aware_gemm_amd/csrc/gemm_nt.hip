// GEMM instantiations for transA='N', transB='T' (A K-contiguous, B K-contiguous):
// the four-wave kernel (tile configurations 256 and 128) and the eight-wave
// ping-pong kernel (256x256).
#include "gemm_kernel.h"
#include "gemm_pp.h"

namespace tgemm {
hipError_t launch_gemm_nt(int cfg, int epi, const GemmParams& p, hipStream_t s) {
  if (cfg == kTilePP) return launch_gemm_pp(epi, p, s);
  return launch_gemm_layout<true, true>(cfg, epi, p, s);
}
}  // namespace tgemm
