// The e4m3fn cast of an fp8 GEMM operand as a pass of its own ("Improve the
// Inductor generated kernel for the pattern of output1 = pointwise(input);
// output2 = transpose(output1)", the example's scale, clamp and cast).
// It writes the cast values, as bf16, to a compact copy in the operand's
// own layout (never a transposed one), with exactly the arithmetic of the
// loader cast (q8_vec), so a GEMM over the copy gives the same bits as one
// that casts on load.  Cast once, an element is not cast again for every
// tile that reads it, and the GEMM reads plain bf16 with its direct
// global->LDS copies.
#include "gemm_kernel.h"
#include "tgemm_internal.h"

namespace tgemm {
namespace {

// One thread: 8 consecutive elements of one row (16-byte load and store).
// X rows are 16-byte aligned (ld % 8 == 0, X aligned) and cols % 8 == 0.
__global__ void __launch_bounds__(256) q8_cast_kernel(const uint16_t* __restrict__ X, int64_t ld,
                                                      int64_t rows, int64_t cols,
                                                      const float* __restrict__ scale,
                                                      uint16_t* __restrict__ out) {
  const int64_t per_row = cols >> 3;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= rows * per_row) return;
  const int64_t r = gid / per_row;
  const int64_t c = (gid - r * per_row) * 8;
  uint4 v = *reinterpret_cast<const uint4*>(X + r * ld + c);
  q8_vec(v, scale[0]);
  *reinterpret_cast<uint4*>(out + r * cols + c) = v;
}

}  // namespace

hipError_t launch_q8_cast(const uint16_t* X, int64_t ld, int64_t rows, int64_t cols,
                          const float* scale, uint16_t* out, hipStream_t s) {
  const int64_t threads = rows * (cols >> 3);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(q8_cast_kernel, dim3((unsigned)blocks), dim3(256), 0, s, X, ld, rows, cols,
                     scale, out);
  return hipGetLastError();
}

}  // namespace tgemm
