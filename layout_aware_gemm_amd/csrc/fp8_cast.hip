// The e4m3fn cast of an fp8 GEMM's operands as a pass of its own ("Improve
// the Inductor generated kernel for the pattern of output1 =
// pointwise(input); output2 = transpose(output1)", the example's scale,
// clamp and cast).
//
// It writes each operand's e4m3fn codes, one byte each, as a K-contiguous
// matrix [Rp][Kp] (R = M for A, N for B) zero-padded to Rp rows and Kp
// columns, which is what the fp8 matrix-core kernel (gemm_f8.hip) reads.
// The arithmetic is the loader cast's (q8_codes), so both routes multiply
// the same e4m3fn values.  An operand stored K-contiguous is cast row by
// row; one stored along M or N is transposed on the way, 16 k by 8 rows per
// thread, so the GEMM never sees the page's second, transposed layout and
// the caller never stores one.  One launch packs both operands: its first
// blocks take A, the rest B.
#include "gemm_kernel.h"
#include "tgemm_internal.h"

namespace tgemm {
namespace {

constexpr int kPackThreads = 256;
constexpr int kRowSeg = 4096;  // codes of one row per wave (rows kernel): 8 loads per lane

struct PackJob {
  const uint16_t* X;
  int64_t ld;
  const float* scale;
  uint8_t* out;
  int64_t threads;  // threads of this job
  int R, K, Rp, Kp;
  int kcontig;      // X is [R][K] (else [K][R])
  uint32_t blocks;  // blocks of this job
};

// K-contiguous operand X [R][K] (row stride ld).  A wave takes a segment of
// kRowSeg codes of one padded row: its loads are 1 KB runs of the row
// (lane l: elements 8l .. 8l+7 of each 512-element part), all issued before
// the first store, its stores 512-byte runs of the codes.  Eight loads in
// flight per lane measured 5% faster on the fp8 linear NN than two.
// Elements at or past K, and rows at or past R, are code 0.
__device__ __forceinline__ void pack_rows(const PackJob& j, int64_t gid) {
  const int lane = (int)(gid & 63);
  const int64_t wv = gid >> 6;
  const int segs = (j.Kp + kRowSeg - 1) / kRowSeg;
  const int64_t r = wv / segs;
  const int e0 = (int)(wv - r * segs) * kRowSeg + 8 * lane;  // first element, part 0
  const float s = j.scale[0];
  const uint16_t* row = j.X + r * j.ld;
  uint8_t* orow = j.out + r * j.Kp;
  constexpr int NH = kRowSeg / 512;
  if (r < j.R && e0 + (NH - 1) * 512 + 8 <= j.K) {
    uint4 v[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) v[h] = *reinterpret_cast<const uint4*>(row + e0 + h * 512);
#pragma unroll
    for (int h = 0; h < NH; ++h) *reinterpret_cast<uint2*>(orow + e0 + h * 512) = q8_codes(v[h], s);
    return;
  }
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int e = e0 + h * 512;
    if (e >= j.Kp) continue;  // (Kp % 128 == 0: a group of 8 is wholly inside or outside)
    uint2 c = make_uint2(0, 0);
    if (r < j.R && e < j.K) c = q8_codes(*reinterpret_cast<const uint4*>(row + e), s);
    *reinterpret_cast<uint2*>(orow + e) = c;
  }
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
// groups of 16 k: it reads 16 stored rows of 128 contiguous bytes and
// writes 64 output rows of 128 contiguous bytes.  Lane bits 0, 2 and 3 give
// the chunk and bits 1, 4 and 5 the group, so lane pairs read 32
// contiguous bytes and even/odd lane pairs write 32 contiguous bytes
// (measured 1-2% faster on the fp8 linear NN than whole 128-byte runs on
// one side only).  Each thread casts its 16 x 8 block and transposes the
// codes in registers.
__device__ __forceinline__ void pack_cols(const PackJob& j, int64_t gid) {
  const int lane = (int)(gid & 63);
  const int64_t wv = gid >> 6;
  const int kblocks = j.Kp >> 7;  // 128 k per wave
  const int64_t rb = wv / kblocks;
  const int kb = (int)(wv - rb * kblocks);
  const int r0 = (int)(rb * 64) + 8 * ((lane & 1) | ((lane >> 1) & 6));
  const int k0 = kb * 128 + 16 * (((lane >> 1) & 1) | ((lane >> 3) & 6));
  const float s = j.scale[0];
  uint32_t lo[16], hi[16];  // codes of rows r0..r0+3 / r0+4..r0+7 at k0 + i
  const uint16_t* src = j.X + (int64_t)k0 * j.ld + r0;
  if (r0 < j.R && k0 + 16 <= j.K) {
    // (R % 8 == 0: the 8 rows are wholly inside or outside)
    uint4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const uint4*>(src + i * j.ld);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint2 c = q8_codes(v[i], s);
      lo[i] = c.x;
      hi[i] = c.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint2 c = make_uint2(0, 0);
      if (r0 < j.R && k0 + i < j.K) c = q8_codes(*reinterpret_cast<const uint4*>(src + i * j.ld), s);
      lo[i] = c.x;
      hi[i] = c.y;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t* w = i < 4 ? lo : hi;
    const int e = i & 3;
    const uint4 o = make_uint4(byte_col(w[0], w[1], w[2], w[3], e),
                               byte_col(w[4], w[5], w[6], w[7], e),
                               byte_col(w[8], w[9], w[10], w[11], e),
                               byte_col(w[12], w[13], w[14], w[15], e));
    *reinterpret_cast<uint4*>(j.out + (int64_t)(r0 + i) * j.Kp + k0) = o;
  }
}

__global__ void __launch_bounds__(kPackThreads) q8_pack_kernel(PackJob a, PackJob b) {
  const bool second = blockIdx.x >= a.blocks;
  const PackJob& j = second ? b : a;
  const int64_t gid =
      (int64_t)(blockIdx.x - (second ? a.blocks : 0u)) * kPackThreads + threadIdx.x;
  if (gid >= j.threads) return;
  if (j.kcontig)
    pack_rows(j, gid);
  else
    pack_cols(j, gid);
}

// The job for one operand, or an error if it breaks the pass's assumptions.
hipError_t make_job(const PackOperand& o, PackJob* j) {
  // (rows: 16-byte vectors along k, K % 8 == 0; cols: along the rows'
  // index, R % 8 == 0)
  if (o.Rp % 64 != 0 || o.Kp % 128 != 0 || o.Rp < o.R || o.Kp < o.K ||
      (o.k_contiguous ? o.K : o.R) % 8 != 0)
    return hipErrorInvalidValue;
  j->X = o.X;
  j->ld = o.ld;
  j->scale = o.scale;
  j->out = o.out;
  j->R = o.R;
  j->K = o.K;
  j->Rp = o.Rp;
  j->Kp = o.Kp;
  j->kcontig = o.k_contiguous ? 1 : 0;
  // rows: one wave per 1024-code segment of a padded row; cols: one thread
  // per 8 rows x 16 k
  j->threads = o.k_contiguous ? (int64_t)o.Rp * ((o.Kp + kRowSeg - 1) / kRowSeg) * 64
                              : (int64_t)(o.Rp >> 3) * (o.Kp >> 4);
  const int64_t blocks = (j->threads + kPackThreads - 1) / kPackThreads;
  if (blocks >= (int64_t(1) << 30)) return hipErrorInvalidValue;
  j->blocks = (uint32_t)blocks;
  return hipSuccess;
}

}  // namespace

hipError_t launch_q8_pack(const PackOperand& a, const PackOperand& b, hipStream_t s) {
  PackJob ja, jb;
  hipError_t e = make_job(a, &ja);
  if (e == hipSuccess) e = make_job(b, &jb);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(q8_pack_kernel, dim3(ja.blocks + jb.blocks), dim3(kPackThreads), 0, s, ja,
                     jb);
  return hipGetLastError();
}

}  // namespace tgemm
