// Measurement aids beside the GEMM path: the shader-clock probe and the
// matrix-core ceiling.
//
// Shader-clock probe.
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

// Matrix-core ceiling.  Every wave issues nothing but MFMAs whose
// operands sit in registers: per iteration, 16 independent 32x32
// accumulator blocks each take one MFMA -- 32x32x16 bf16 (KIND 0, 524288
// flop per wave and iteration) or 32x32x64 on fp8 e4m3fn codes (KIND 1,
// 2097152) -- block q from operands a[q % 4] and b[q / 4], so no result
// feeds an operand and no two blocks compute the same thing (the compiler
// would merge them).  It is the GEMM loops' matrix-core work without loads,
// LDS or barriers: the rate they could reach at the clock the chip holds
// under such work.  Operands have random-looking bits derived from the
// thread and register index: finite bf16 values (sign, 7 mantissa bits,
// exponents 2^-7 .. 2^0) or e4m3fn codes with the top exponent bit clear
// (never NaN).  Lane 0 of each wave writes element 0 of block 0 to
// out[block * 4 + wave].
typedef __bf16 cl_bf16x8_t __attribute__((ext_vector_type(8)));
typedef int cl_i32x8_t __attribute__((ext_vector_type(8)));
typedef float cl_f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t ceiling_hash(uint32_t seed, int e) {
  uint32_t h = (seed + 0x9e3779b9u * (uint32_t)(e + 1)) * 0x85ebca6bu;
  h ^= h >> 13;
  return h;
}

template <int KIND>
struct CeilingOp;
template <>
struct CeilingOp<0> {
  typedef cl_bf16x8_t type;
  static __device__ __forceinline__ type make(uint32_t seed) {
    type v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = ceiling_hash(seed, e);
      // sign | exponent 120..127 | 7 mantissa bits
      const uint16_t bits =
          (uint16_t)((h & 0x8000u) | ((120u + ((h >> 8) & 7u)) << 7) | (h & 0x7fu));
      v[e] = __builtin_bit_cast(__bf16, bits);
    }
    return v;
  }
  static __device__ __forceinline__ cl_f32x16_t mma(const type& a, const type& b,
                                                    const cl_f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct CeilingOp<1> {
  typedef cl_i32x8_t type;
  static __device__ __forceinline__ type make(uint32_t seed) {
    type v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (int)(ceiling_hash(seed, e) & 0xb7b7b7b7u);
    return v;
  }
  static __device__ __forceinline__ cl_f32x16_t mma(const type& a, const type& b,
                                                    const cl_f32x16_t& c) {
    // format 0 (e4m3fn) for both operands; zero scales: the unscaled MFMA
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

template <int KIND>
__global__ void __launch_bounds__(256, 1) mfma_ceiling_kernel(int64_t iters, float* out) {
  using Op = CeilingOp<KIND>;
  const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 8u;
  typename Op::type a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = Op::make(seed + i);
    b[i] = Op::make(seed + 4 + i);
  }
  cl_f32x16_t acc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[q][i] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = Op::mma(a[q & 3], b[q >> 2], acc[q]);
  }
  float r = acc[0][0], keep = 0.f;
#pragma unroll
  for (int q = 1; q < 16; ++q) keep += acc[q][0];
  // (every block feeds the result, so none is dropped)
  if (keep == 12345.f) r += 1.f;
  if ((threadIdx.x & 63u) == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = r;
}

}  // namespace
}  // namespace tgemm

extern "C" int tgemm_mfma_ceiling(int kind, int64_t iters, int blocks, float* out,
                                  void* stream) {
  if ((kind != 0 && kind != 1) || iters < 1 || iters > 100000000 || blocks < 1 ||
      blocks > 65536 || out == nullptr || (reinterpret_cast<uintptr_t>(out) & 3) != 0)
    return TGEMM_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // (96 KB of LDS reserved, unused: one workgroup per compute unit)
  if (kind == 0)
    hipLaunchKernelGGL(tgemm::mfma_ceiling_kernel<0>, dim3(blocks), dim3(256), 96 * 1024, st,
                       iters, out);
  else
    hipLaunchKernelGGL(tgemm::mfma_ceiling_kernel<1>, dim3(blocks), dim3(256), 96 * 1024, st,
                       iters, out);
  return hipGetLastError() == hipSuccess ? TGEMM_OK : TGEMM_ERR_HIP;
}

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
