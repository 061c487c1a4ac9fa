// Shader-clock probe, a measurement aid beside the GEMM path.
//
// MI355X lowers its shader clock under sustained matrix-core load, so a
// kernel's rate at the clock it ran at can differ from its rate against the
// nominal 2.4 GHz peak.  One wave reads the shader-cycle counter
// (s_memtime) and the constant-rate counter (s_memrealtime), polls the
// constant-rate counter until it has advanced by `ticks` (with a fixed cap
// on the number of polls, so the wave always exits), and reads both again.
// The shader clock over the wait is cycles * rate / ticks.  Enqueued right
// after a timed region, it reads the clock that region ended at.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tgemm.h"

namespace tgemm {
namespace {

constexpr int kMaxPolls = 1 << 22;

__global__ void __launch_bounds__(64) clock_probe_kernel(uint64_t* out, uint64_t ticks,
                                                         uint64_t rate_hz) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  uint64_t r1 = r0;
  for (int i = 0; i < kMaxPolls && r1 - r0 < ticks; ++i) r1 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
    out[2] = rate_hz;
  }
}

}  // namespace
}  // namespace tgemm

extern "C" int tgemm_clock_probe(int64_t ticks, uint64_t* out_ticks, void* stream) {
  if (ticks < 1 || ticks > 10000000 || out_ticks == nullptr ||
      (reinterpret_cast<uintptr_t>(out_ticks) & 7) != 0)
    return TGEMM_ERR_INVALID_ARG;
  // the rate of the device the stream belongs to (the null stream: the
  // current device)
  int dev = 0, khz = 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if ((st == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(st, &dev)) != hipSuccess)
    return TGEMM_ERR_HIP;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
    return TGEMM_ERR_HIP;
  hipLaunchKernelGGL(tgemm::clock_probe_kernel, dim3(1), dim3(64), 0, st, out_ticks,
                     (uint64_t)ticks, (uint64_t)khz * 1000u);
  return hipGetLastError() == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
}
