// Degenerate K=1 matmuls as pointwise kernels (no matrix cores).
//
// "Schedule a small matmul op as a reduction (or pointwise) op": with K=1
// the matmul is a broadcast of both operands, one elementwise multiply and
// a squeeze, so it can live in the same kernel as the pointwise work around
// it.  For the RoPE table the listing widens the [64] inverse frequencies
// and casts the int64 positions to fp32, multiplies, permutes to
// [positions, 64], duplicates the last dimension to 128 and takes cos (and,
// for the second declared output, sin) before casting to bf16.  Here the
// permute is free (positions are operand A, so the product is produced
// directly as [positions, 64]; fp32 multiplication commutes exactly), the
// duplication is a second store of the same value, and everything from the
// int64 load to the bf16 stores is one kernel.
#include "bf16_cvt.h"
#include "tgemm_internal.h"

namespace tgemm {

namespace {


// Largest |t| the reduced-argument sin/cos below is used for; beyond it
// (positions past 65536 at the unit frequency, or infinities) the library
// sincosf with its large-argument reduction is called instead.
constexpr float kFastTrigLimit = 65536.0f;

// sin(t) and cos(t) for |t| <= kFastTrigLimit, about 24 VALU operations.
// Cody and Waite's argument reduction: t = k*pi/2 + r with k = rint(t*2/pi)
// and pi/2 split into three fp32 parts c1 + c2 + c3 (c1 = pi/2 rounded to
// fp32, c2 = the remainder rounded to fp32, c3 = the remainder of that;
// what is left is 1.1e-23), subtracted with fused multiply-adds so each
// step rounds once: |r| <= pi/4 + 0.01 and the reduction error is below
// 1.2e-7 for every |k| <= 41722.  Then the Taylor polynomials of sin (to
// r^7) and cos (to r^8), whose first omitted terms are below 3.4e-7 and
// 2.8e-8 on that interval -- far below the 2^-9 relative step of the bf16
// results -- and the quadrant k mod 4 selects and signs them: sin(t) = (sin r, cos r, -sin r, -cos r), cos(t) = (cos r, -sin r,
// -cos r, sin r) for k mod 4 = 0, 1, 2, 3.
__device__ __forceinline__ void sincos_reduced(float t, float& sn, float& cs) {
  const float kf = rintf(t * 0x1.45f306p-1f);              // 2/pi
  float r = fmaf(-kf, 0x1.921fb6p+0f, t);                 // c1
  r = fmaf(-kf, -0x1.777a5cp-25f, r);                     // c2
  r = fmaf(-kf, -0x1.ee59dap-50f, r);                     // c3
  const float r2 = r * r;
  float ps = fmaf(r2, -0x1.a01a02p-13f, 0x1.111112p-7f);  // -1/7!, 1/5!
  ps = fmaf(r2, ps, -0x1.555556p-3f);                     // -1/3!
  const float sr = fmaf(r * r2, ps, r);
  float pc = fmaf(r2, 0x1.a01a02p-16f, -0x1.6c16c2p-10f);  // 1/8!, -1/6!
  pc = fmaf(r2, pc, 0x1.555556p-5f);                      // 1/4!
  pc = fmaf(r2, pc, -0.5f);                               // -1/2!
  const float cr = fmaf(r2, pc, 1.0f);
  const int q = (int)kf;
  const float a = (q & 1) ? cr : sr;
  const float b = (q & 1) ? sr : cr;
  sn = __uint_as_float(__float_as_uint(a) ^ ((uint32_t)(q & 2) << 30));
  cs = __uint_as_float(__float_as_uint(b) ^ ((uint32_t)((q + 1) & 2) << 30));
}

__device__ __forceinline__ void sincos_t(float t, float& sn, float& cs) {
  if (fabsf(t) <= kFastTrigLimit) {
    sincos_reduced(t, sn, cs);
  } else {
    sincosf(t, &sn, &cs);
  }
}

// Rows per thread of the RoPE kernel.  A thread loads all RPT positions
// first and then computes and stores each row: the position loads overlap
// each other and the trig of the earlier rows.  When the column groups of
// a row divide the 256 threads of a workgroup (spb = 256 / groups row
// slots per workgroup), workgroup b writes the RPT*spb consecutive rows
// from b*RPT*spb on, thread slot s its rows s, s + spb, ...: each
// workgroup fills one contiguous block of both tables, and the lanes of one
// store instruction still cover consecutive rows.  Otherwise (spb = 0) a
// thread takes RPT rows that are `slots` rows apart.
constexpr int kRopeRows = 2;

// One thread per (row slot, group of 8 columns); `gid` is the thread's index
// in the table's part of the grid.
template <int RPT>
__device__ __forceinline__ void rope_table_part(
    uint32_t gid, const int64_t* __restrict__ pos, int64_t spos, const float* __restrict__ invf,
    int64_t sinv, int M, int N, uint16_t* __restrict__ cos_out, uint16_t* __restrict__ sin_out,
    int64_t ldc, int vec_ok, uint32_t spb) {
  // (the grid has fewer than 2^32 threads, so 32-bit index arithmetic)
  const uint32_t groups = (uint32_t)(N + 7) >> 3;
  const uint32_t slots = spb ? ((uint32_t)M + spb * RPT - 1) / (spb * RPT) * spb
                            : ((uint32_t)M + RPT - 1) / RPT;
  const uint32_t rs = gid / groups;
  if (rs >= slots) return;
  const int c0 = (int)(gid - rs * groups) * 8;
  float pf[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int64_t row = spb ? (int64_t)(rs / spb) * spb * RPT + (int64_t)j * spb + rs % spb
                             : (int64_t)rs + (int64_t)j * slots;
    const int64_t pv = row < M ? pos[row * spos] : 0;
    // int64 -> fp32, rounded to nearest even (exact below 2^24); one
    // instruction when the position fits in 32 bits
    pf[j] = pv == (int64_t)(int32_t)pv ? (float)(int32_t)pv : (float)pv;
  }
  if (vec_ok && c0 + 8 <= N) {
    const float4 f0 = *reinterpret_cast<const float4*>(invf + c0);
    const float4 f1 = *reinterpret_cast<const float4*>(invf + c0 + 4);
    const float fr[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int64_t row = spb ? (int64_t)(rs / spb) * spb * RPT + (int64_t)j * spb + rs % spb
                             : (int64_t)rs + (int64_t)j * slots;
      if (row >= M) break;
      float t[8], sv8[8], cv8[8], m = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        t[e] = __fmul_rn(pf[j], fr[e]);  // one fp32 multiply, never contracted
        m = fmaxf(m, fabsf(t[e]));
      }
      if (m <= kFastTrigLimit) {  // (NaN arguments take this branch and stay NaN)
#pragma unroll
        for (int e = 0; e < 8; ++e) sincos_reduced(t[e], sv8[e], cv8[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) sincosf(t[e], &sv8[e], &cv8[e]);
      }
      uint32_t cw[4], sw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        cw[q] = pack_bf16x2(cv8[2 * q], cv8[2 * q + 1]);
        sw[q] = pack_bf16x2(sv8[2 * q], sv8[2 * q + 1]);
      }
      uint16_t* co = cos_out + row * ldc;
      uint16_t* so = sin_out + row * ldc;
      // streaming stores: the tables are written once and not read back here
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 cq = {cw[0], cw[1], cw[2], cw[3]}, sq = {sw[0], sw[1], sw[2], sw[3]};
      __builtin_nontemporal_store(cq, reinterpret_cast<u32x4*>(co + c0));
      __builtin_nontemporal_store(cq, reinterpret_cast<u32x4*>(co + c0 + N));
      __builtin_nontemporal_store(sq, reinterpret_cast<u32x4*>(so + c0));
      __builtin_nontemporal_store(sq, reinterpret_cast<u32x4*>(so + c0 + N));
    }
  } else {
    for (int j = 0; j < RPT; ++j) {
      const int64_t row = spb ? (int64_t)(rs / spb) * spb * RPT + (int64_t)j * spb + rs % spb
                             : (int64_t)rs + (int64_t)j * slots;
      if (row >= M) break;
      uint16_t* co = cos_out + row * ldc;
      uint16_t* so = sin_out + row * ldc;
      for (int e = 0; e < 8 && c0 + e < N; ++e) {
        const int c = c0 + e;
        float sv, cv;
        sincos_t(__fmul_rn(pf[j], invf[c * sinv]), sv, cv);
        const uint16_t cb = to_bf16(cv), sb = to_bf16(sv);
        co[c] = cb;
        co[c + N] = cb;
        so[c] = sb;
        so[c + N] = sb;
      }
    }
  }
}

template <int RPT>
__global__ void __launch_bounds__(256) k1_rope_kernel(
    const int64_t* __restrict__ pos, int64_t spos, const float* __restrict__ invf, int64_t sinv,
    int M, int N, uint16_t* __restrict__ cos_out, uint16_t* __restrict__ sin_out, int64_t ldc,
    int vec_ok, uint32_t spb) {
  rope_table_part<RPT>(blockIdx.x * blockDim.x + threadIdx.x, pos, spos, invf, sinv, M, N,
                       cos_out, sin_out, ldc, vec_ok, spb);
}

// The query part of the RoPE region ("Schedule a small matmul op as a
// reduction (or pointwise) op", the %kernel_math listing: the [P, H*D] bf16
// query viewed as [P, H, D], permuted to [H, P, D] and cast to fp32).  One
// thread per 8 consecutive elements of a query row: a 16-byte load, the
// exact bf16 -> fp32 widening, and two 16-byte streaming stores into the
// head-major fp32 output.  The 64 lanes of a wave read 1 KB of one query row
// and write it as 512-byte runs of the output rows of consecutive heads.
__device__ __forceinline__ void rope_query_part(uint64_t g, const uint16_t* __restrict__ q,
                                                int64_t ldq, int64_t P, int64_t H, int64_t D,
                                                float* __restrict__ out, int vec_ok) {
  const int64_t per_row = (H * D + 7) >> 3;
  const int64_t p = (int64_t)(g / (uint64_t)per_row);
  if (p >= P) return;
  const int64_t c0 = (int64_t)(g - (uint64_t)p * per_row) * 8;
  const uint16_t* src = q + p * ldq + c0;
  if (vec_ok && c0 + 8 <= H * D) {
    // D % 8 == 0: the 8 elements belong to one head
    const int64_t h = c0 / D, d = c0 - h * D;
    const uint4 v = *reinterpret_cast<const uint4*>(src);
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const f32x4v lo = {from_bf16(v.x & 0xffffu), from_bf16(v.x >> 16), from_bf16(v.y & 0xffffu),
                       from_bf16(v.y >> 16)};
    const f32x4v hi = {from_bf16(v.z & 0xffffu), from_bf16(v.z >> 16), from_bf16(v.w & 0xffffu),
                       from_bf16(v.w >> 16)};
    float* dst = out + (h * P + p) * D + d;
    __builtin_nontemporal_store(lo, reinterpret_cast<f32x4v*>(dst));
    __builtin_nontemporal_store(hi, reinterpret_cast<f32x4v*>(dst + 4));
  } else {
    for (int e = 0; e < 8 && c0 + e < H * D; ++e) {
      const int64_t c = c0 + e, h = c / D, d = c - h * D;
      out[(h * P + p) * D + d] = from_bf16(src[e]);
    }
  }
}

// The region in one launch: workgroups [0, tbl_blocks) build the cos / sin
// tables of the positions (the K = 1 product and its epilogue), the rest
// widen and permute the query.  The two parts share no data.
__global__ void __launch_bounds__(256) rope_region_kernel(
    const int64_t* __restrict__ pos, int64_t spos, const float* __restrict__ invf, int P, int F,
    uint16_t* __restrict__ cos_out, uint16_t* __restrict__ sin_out, int64_t ldc, int vec_tbl,
    uint32_t spb, uint32_t tbl_blocks, const uint16_t* __restrict__ q, int64_t ldq, int64_t H,
    int64_t D, float* __restrict__ q_out, int vec_q) {
  if (blockIdx.x < tbl_blocks) {
    rope_table_part<kRopeRows>(blockIdx.x * blockDim.x + threadIdx.x, pos, spos, invf, 1, P, F,
                               cos_out, sin_out, ldc, vec_tbl, spb);
  } else {
    const uint64_t g = (uint64_t)(blockIdx.x - tbl_blocks) * blockDim.x + threadIdx.x;
    rope_query_part(g, q, ldq, P, H, D, q_out, vec_q);
  }
}

// C[m, n] = a[m] * b[n], fp32 inputs, one fp32 multiply.
__global__ void __launch_bounds__(256) k1_outer_f32_kernel(const float* __restrict__ a, int64_t sa,
                                                           const float* __restrict__ b, int64_t sb,
                                                           int M, int N, float* __restrict__ C,
                                                           int64_t ldc) {
  const int groups = (N + 3) >> 2;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / groups;
  if (row >= M) return;
  const int c0 = (int)(gid - row * groups) * 4;
  const float av = a[row * sa];
  float* out = C + row * ldc;
  for (int e = 0; e < 4 && c0 + e < N; ++e) out[c0 + e] = __fmul_rn(av, b[(int64_t)(c0 + e) * sb]);
}

// K = 1 with bf16 operands and a store epilogue: the bf16 x bf16 product is
// exact in fp32, then stored as fp32 or rounded to bf16.
__global__ void __launch_bounds__(256) k1_outer_bf16_kernel(
    const uint16_t* __restrict__ a, int64_t sa, const uint16_t* __restrict__ b, int64_t sb, int M,
    int N, void* __restrict__ C, int64_t ldc, int out_f32) {
  const int groups = (N + 3) >> 2;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / groups;
  if (row >= M) return;
  const int c0 = (int)(gid - row * groups) * 4;
  const float av = from_bf16(a[row * sa]);
  for (int e = 0; e < 4 && c0 + e < N; ++e) {
    const float v = __fmul_rn(av, from_bf16(b[(int64_t)(c0 + e) * sb]));
    if (out_f32)
      reinterpret_cast<float*>(C)[row * ldc + c0 + e] = v;
    else
      reinterpret_cast<uint16_t*>(C)[row * ldc + c0 + e] = to_bf16(v);
  }
}

// K = 1 with the cross-entropy epilogue: row m's logits are y[n] = a[m] *
// b[n] (bf16 operands; the product is exact in fp32), so the row reduction
// needs no matrix cores either.  One workgroup per row.  Pass 1: the row
// max; pass 2: the sum of exp(y - max); each thread walks a strided share
// of the columns in ascending order and the 256 thread values are folded
// by a fixed tree in LDS, so the result is deterministic.  lse = max +
// ln(sum), loss = lse - y[label] (NaN for a label outside [0, N)).  With a
// gradient buffer, pass 3 writes bf16(exp(y - lse) - [n == label]).  A NaN
// logit makes the sum, and so the loss and the gradient row, NaN.
constexpr int kCeK1Threads = 256;
constexpr float kCeLog2e = 1.4426950408889634f;
constexpr float kCeLn2 = 0.6931471805599453f;

__device__ __forceinline__ float block_fold(float v, float* red, bool is_max) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
#pragma unroll
  for (int o = kCeK1Threads / 2; o > 0; o >>= 1) {
    if (t < o) red[t] = is_max ? fmaxf(red[t], red[t + o]) : red[t] + red[t + o];
    __syncthreads();
  }
  const float r = red[0];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(kCeK1Threads) k1_ce_kernel(
    const uint16_t* __restrict__ a, int64_t sa, const uint16_t* __restrict__ b, int64_t sb, int N,
    const int32_t* __restrict__ labels, float* __restrict__ loss, uint16_t* __restrict__ grad,
    int64_t ldg) {
  __shared__ float red[kCeK1Threads];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const float av = from_bf16(a[row * sa]);
  float mx = -INFINITY;
  for (int n = t; n < N; n += kCeK1Threads)
    mx = fmaxf(mx, __fmul_rn(av, from_bf16(b[(int64_t)n * sb])));
  mx = block_fold(mx, red, true);
  float sum = 0.f;
  for (int n = t; n < N; n += kCeK1Threads)
    sum += exp2f((__fmul_rn(av, from_bf16(b[(int64_t)n * sb])) - mx) * kCeLog2e);
  sum = block_fold(sum, red, false);
  const float lse = mx + log2f(sum) * kCeLn2;
  const int lab = labels[row];
  const bool valid = lab >= 0 && lab < N;
  if (t == 0)
    loss[row] = valid ? lse - __fmul_rn(av, from_bf16(b[(int64_t)lab * sb]))
                      : __int_as_float(0x7fc00000);
  if (grad == nullptr) return;
  uint16_t* g = grad + row * ldg;
  for (int n = t; n < N; n += kCeK1Threads) {
    const float y = __fmul_rn(av, from_bf16(b[(int64_t)n * sb]));
    g[n] = to_bf16(exp2f((y - lse) * kCeLog2e) - (n == lab ? 1.f : 0.f));
  }
}

inline unsigned grid_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

}  // namespace

struct RopeGeom {
  int vec_ok;
  uint32_t spb;
  int64_t threads;
};

static RopeGeom rope_geom(const float* invf, int64_t sinv, int M, int N, const uint16_t* cos_out,
                   const uint16_t* sin_out, int64_t ldc) {
  RopeGeom g;
  g.vec_ok = sinv == 1 && (reinterpret_cast<uintptr_t>(invf) & 15) == 0 &&
             (reinterpret_cast<uintptr_t>(cos_out) & 15) == 0 &&
             (reinterpret_cast<uintptr_t>(sin_out) & 15) == 0 && ldc % 8 == 0 && N % 8 == 0;
  const int64_t groups = (N + 7) / 8;
  g.spb = groups <= 256 && 256 % groups == 0 ? (uint32_t)(256 / groups) : 0;
  const int64_t slots = g.spb ? ((int64_t)M + g.spb * kRopeRows - 1) / (g.spb * kRopeRows) * g.spb
                              : ((int64_t)M + kRopeRows - 1) / kRopeRows;
  g.threads = slots * groups;
  return g;
}

hipError_t launch_k1_rope(const int64_t* pos, int64_t spos, const float* invf, int64_t sinv,
                          int M, int N, uint16_t* cos_out, uint16_t* sin_out, int64_t ldc,
                          hipStream_t s) {
  const RopeGeom g = rope_geom(invf, sinv, M, N, cos_out, sin_out, ldc);
  if (g.threads >= (int64_t(1) << 32)) return hipErrorInvalidValue;  // 32-bit thread index
  hipLaunchKernelGGL(k1_rope_kernel<kRopeRows>, dim3(grid_for(g.threads)), dim3(256), 0, s, pos,
                     spos, invf, sinv, M, N, cos_out, sin_out, ldc, g.vec_ok, g.spb);
  return hipGetLastError();
}

hipError_t launch_rope_region(const uint16_t* q, int64_t ldq, int64_t P, int64_t H, int64_t D,
                              const int64_t* pos, int64_t spos, const float* invf,
                              uint16_t* cos_out, uint16_t* sin_out, int64_t ldc, float* q_out,
                              hipStream_t s) {
  const int F = (int)(D / 2);
  const RopeGeom g = rope_geom(invf, 1, (int)P, F, cos_out, sin_out, ldc);
  const int64_t tbl_blocks = (g.threads + 255) / 256;
  const int64_t q_threads = P * ((H * D + 7) / 8);
  const int64_t q_blocks = (q_threads + 255) / 256;
  if (g.threads >= (int64_t(1) << 32) || tbl_blocks + q_blocks >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  const int vec_q = (reinterpret_cast<uintptr_t>(q) & 15) == 0 && ldq % 8 == 0 && D % 8 == 0 &&
                    (reinterpret_cast<uintptr_t>(q_out) & 15) == 0;
  hipLaunchKernelGGL(rope_region_kernel, dim3((unsigned)(tbl_blocks + q_blocks)), dim3(256), 0, s,
                     pos, spos, invf, (int)P, F, cos_out, sin_out, ldc, g.vec_ok, g.spb,
                     (uint32_t)tbl_blocks, q, ldq, H, D, q_out, vec_q);
  return hipGetLastError();
}

hipError_t launch_k1_outer_f32(const float* a, int64_t sa, const float* b, int64_t sb, int M,
                               int N, float* C, int64_t ldc, hipStream_t s) {
  const int64_t threads = (int64_t)M * ((N + 3) / 4);
  hipLaunchKernelGGL(k1_outer_f32_kernel, dim3(grid_for(threads)), dim3(256), 0, s, a, sa, b, sb,
                     M, N, C, ldc);
  return hipGetLastError();
}

hipError_t launch_k1_outer_bf16(const uint16_t* a, int64_t sa, const uint16_t* b, int64_t sb,
                                int M, int N, void* C, int64_t ldc, bool out_f32, hipStream_t s) {
  const int64_t threads = (int64_t)M * ((N + 3) / 4);
  hipLaunchKernelGGL(k1_outer_bf16_kernel, dim3(grid_for(threads)), dim3(256), 0, s, a, sa, b, sb,
                     M, N, C, ldc, out_f32 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_k1_ce(const uint16_t* a, int64_t sa, const uint16_t* b, int64_t sb, int M,
                        int N, const int32_t* labels, float* loss, uint16_t* grad, int64_t ldg,
                        hipStream_t s) {
  hipLaunchKernelGGL(k1_ce_kernel, dim3((unsigned)M), dim3(kCeK1Threads), 0, s, a, sa, b, sb, N,
                     labels, loss, grad, ldg);
  return hipGetLastError();
}

}  // namespace tgemm
