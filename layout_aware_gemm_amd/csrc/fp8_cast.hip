// The e4m3fn cast of an fp8 GEMM operand as a pass of its own ("Improve the
// Inductor generated kernel for the pattern of output1 = pointwise(input);
// output2 = transpose(output1)", the example's scale, clamp and cast).
//
// It writes the operand's e4m3fn codes, one byte each, as a K-contiguous
// matrix [Rp][Kp] (R = M for A, N for B) zero-padded to Rp rows and Kp
// columns, which is what the fp8 matrix-core kernel (gemm_f8.hip) reads.
// The arithmetic is the loader cast's (q8_codes), so both routes multiply
// the same e4m3fn values.  An operand stored K-contiguous is cast row by
// row; one stored along M or N is transposed on the way, 16 k by 8 rows
// per thread, so the GEMM never sees the page's second, transposed layout
// and the caller never stores one.
#include "gemm_kernel.h"
#include "tgemm_internal.h"

namespace tgemm {
namespace {

// K-contiguous operand X [R][K] (row stride ld): thread = 16 consecutive
// codes (two 16-byte loads, one 16-byte store) of one padded row.
__global__ void __launch_bounds__(256) q8_pack_rows_kernel(const uint16_t* __restrict__ X,
                                                           int64_t ld, int R, int K,
                                                           const float* __restrict__ scale,
                                                           uint8_t* __restrict__ out, int Kp,
                                                           int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int per_row = Kp >> 4;
  const int64_t r = gid / per_row;
  const int k = (int)(gid - r * per_row) * 16;
  const float s = scale[0];
  uint2 c[2] = {make_uint2(0, 0), make_uint2(0, 0)};
#pragma unroll
  for (int h = 0; h < 2; ++h)
    if (r < R && k + 8 * h < K)  // K % 8 == 0: a vector is wholly inside or outside
      c[h] = q8_codes(*reinterpret_cast<const uint4*>(X + r * ld + k + 8 * h), s);
  *reinterpret_cast<uint4*>(out + r * Kp + k) = make_uint4(c[0].x, c[0].y, c[1].x, c[1].y);
}

// Bytes e of the four registers w0..w3, as one register (w0's in byte 0).
__device__ __forceinline__ uint32_t byte_col(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                             int e) {
  const int sh = 8 * e;
  return ((w0 >> sh) & 0xffu) | (((w1 >> sh) & 0xffu) << 8) | (((w2 >> sh) & 0xffu) << 16) |
         (((w3 >> sh) & 0xffu) << 24);
}

// Operand stored contiguous along its rows' index: X [K][R] (row stride ld,
// element (k, r) at X + k*ld + r).  A wave covers 8 chunks of 8 r by 8
// groups of 16 k (lane = 8 * group + chunk): it reads 16 stored rows of
// 128 contiguous bytes and writes 64 output rows of 128 contiguous bytes.
// Each thread casts its 16 x 8 block and transposes the codes in registers.
__global__ void __launch_bounds__(256) q8_pack_cols_kernel(const uint16_t* __restrict__ X,
                                                           int64_t ld, int R, int K,
                                                           const float* __restrict__ scale,
                                                           uint8_t* __restrict__ out, int Kp,
                                                           int64_t total) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int lane = (int)(gid & 63);
  const int64_t wv = gid >> 6;
  const int kblocks = Kp >> 7;  // 128 k per wave
  const int64_t rb = wv / kblocks;
  const int kb = (int)(wv - rb * kblocks);
  const int r0 = (int)(rb * 64) + 8 * (lane & 7);
  const int k0 = kb * 128 + 16 * (lane >> 3);
  const float s = scale[0];
  uint32_t lo[16], hi[16];  // codes of rows r0..r0+3 / r0+4..r0+7 at k0 + j
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint2 c = make_uint2(0, 0);
    if (r0 < R && k0 + j < K)  // R % 8 == 0: the 8 rows are wholly inside or outside
      c = q8_codes(*reinterpret_cast<const uint4*>(X + (int64_t)(k0 + j) * ld + r0), s);
    lo[j] = c.x;
    hi[j] = c.y;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t* w = i < 4 ? lo : hi;
    const int e = i & 3;
    const uint4 v = make_uint4(byte_col(w[0], w[1], w[2], w[3], e),
                               byte_col(w[4], w[5], w[6], w[7], e),
                               byte_col(w[8], w[9], w[10], w[11], e),
                               byte_col(w[12], w[13], w[14], w[15], e));
    *reinterpret_cast<uint4*>(out + (int64_t)(r0 + i) * Kp + k0) = v;
  }
}

}  // namespace

hipError_t launch_q8_pack(const uint16_t* X, int64_t ld, bool k_contiguous, int R, int K,
                          const float* scale, uint8_t* out, int Rp, int Kp, hipStream_t s) {
  // (rows kernel: 16-byte vectors along k, K % 8 == 0; cols kernel: along
  // the rows' index, R % 8 == 0)
  if (Rp % 64 != 0 || Kp % 128 != 0 || Rp < R || Kp < K || (k_contiguous ? K : R) % 8 != 0)
    return hipErrorInvalidValue;
  // one thread per 16 codes of a row, or per 8 rows x 16 k
  const int64_t total = k_contiguous ? (int64_t)Rp * (Kp >> 4) : (int64_t)(Rp >> 3) * (Kp >> 4);
  const int64_t blocks = (total + 255) / 256;
  if (blocks >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  if (k_contiguous)
    hipLaunchKernelGGL(q8_pack_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, X, ld, R, K,
                       scale, out, Kp, total);
  else
    hipLaunchKernelGGL(q8_pack_cols_kernel, dim3((unsigned)blocks), dim3(256), 0, s, X, ld, R, K,
                       scale, out, Kp, total);
  return hipGetLastError();
}

}  // namespace tgemm
