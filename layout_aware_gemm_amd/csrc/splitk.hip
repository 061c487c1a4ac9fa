// Split-K sum: the GEMM kernel leaves one fp32 partial product per K chunk,
// ws[q][M][N]; this pass adds them in chunk order q = 0, 1, ..., split-1 --
// a fixed order, so the result does not depend on which chunk finished
// first -- and writes C in bf16 (round to nearest even) or fp32.
//
// A separate pass rather than a last-arriving workgroup: each XCD has its
// own L2, so an in-kernel hand-off needs a device-scope release (an L2
// write-back) in every workgroup and an acquire (an L2 invalidate) in the
// last; the kernel boundary gives the same visibility once per launch.
#include "bf16_cvt.h"
#include "tgemm_internal.h"

namespace tgemm {

namespace {

// One thread: 8 consecutive columns of one row (two 16-byte loads per
// chunk when the rows are 16-byte aligned).
__global__ void __launch_bounds__(256) splitk_sum_kernel(const float* __restrict__ ws, int split,
                                                         int M, int N, void* __restrict__ C,
                                                         int64_t ldc, int out_f32, int vec_in,
                                                         int vec_out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int groups = (N + 7) >> 3;
  const int64_t row = gid / groups;
  if (row >= M) return;
  const int c0 = (int)(gid - row * groups) * 8;
  const int64_t slice = (int64_t)M * N;
  const float* src = ws + row * N + c0;
  const bool full = c0 + 8 <= N;
  float v[8];
  if (vec_in && full) {
    float4 a = *reinterpret_cast<const float4*>(src);
    float4 b = *reinterpret_cast<const float4*>(src + 4);
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
    for (int q = 1; q < split; ++q) {
      a = *reinterpret_cast<const float4*>(src + q * slice);
      b = *reinterpret_cast<const float4*>(src + q * slice + 4);
      v[0] += a.x, v[1] += a.y, v[2] += a.z, v[3] += a.w;
      v[4] += b.x, v[5] += b.y, v[6] += b.z, v[7] += b.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = c0 + e < N ? src[e] : 0.f;
    for (int q = 1; q < split; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (c0 + e < N) v[e] += src[q * slice + e];
  }
  if (out_f32) {
    float* out = static_cast<float*>(C) + row * ldc + c0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c0 + e < N) out[e] = v[e];
    return;
  }
  uint16_t* out = static_cast<uint16_t*>(C) + row * ldc + c0;
  if (vec_out && full) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
    *reinterpret_cast<uint4*>(out) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c0 + e < N) out[e] = to_bf16(v[e]);
  }
}

}  // namespace

hipError_t launch_splitk_sum(const float* ws, int split, int M, int N, void* C, int64_t ldc,
                             bool out_f32, hipStream_t s) {
  const int64_t threads = (int64_t)M * ((N + 7) / 8);
  const int64_t blocks = (threads + 255) / 256;
  const int vec_in = (N % 4) == 0 && (reinterpret_cast<uintptr_t>(ws) & 15) == 0;
  const int vec_out = (ldc % 8) == 0 && (reinterpret_cast<uintptr_t>(C) & 15) == 0;
  hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ws, split, M, N,
                     C, ldc, out_f32 ? 1 : 0, vec_in, vec_out);
  return hipGetLastError();
}

}  // namespace tgemm
