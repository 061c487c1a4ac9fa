// Cross-entropy combine and gradient fix-up kernels.
//
// "Allow reductions in matmul epilogues" asks whether a row-wise reduction
// can run when the matmul is computed tile by tile; the answer given there
// is a grid reduction (atomics or semaphores), and a cooperative launch
// when the reduced value feeds back into other epilogue outputs.  Here the
// GEMM epilogue leaves one (block max, block sum) pair per row and per
// column block; `ce_combine` folds those pairs per row in a fixed order (so
// the result is deterministic), and the gradient,
// which needs the row's final logsumexp, is finished by `ce_grad_fixup`
// in a second pass instead of a cooperative launch.
#include "bf16_cvt.h"
#include "ce_grad.h"
#include "tgemm_internal.h"

namespace tgemm {

namespace {

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;

__device__ __forceinline__ float exp_f(float x) { return exp2f(x * kLog2eF); }


// Workgroup = 64 rows x 16 parts; wave q takes part q, the blocks t = q,
// q+16, q+32, ..., for 64 consecutive rows (one 256-byte load per block).
// The first kCombCache blocks of a part (every block up to N = 32768 with
// 128-column blocks) are loaded at once, both arrays unconditionally, and
// kept in registers for both passes: the kernel waits for memory about
// once instead of once per block.  Two passes instead of a chain of
// pairwise merges: the row max over every non-empty block, then the sum of
// s_t * exp(m_t - max), whose exponentials are independent of each other.  Each part adds its blocks in ascending t
// and the sixteen part sums are added in ascending part order: a fixed order,
// so the result is deterministic.  A block with s == 0 holds no column and
// is skipped; a block whose sum is NaN (a NaN logit, or exp(inf - inf))
// makes the row's logsumexp NaN, and with it the loss and the gradient row.
// This is the pairwise (m, s) (+) (m', s') = (M, s e^{m-M} + s' e^{m'-M})
// merge unrolled: any order of merges gives the same max and, up to
// rounding, the same sum.
constexpr int kCombRows = 64, kCombParts = 16, kCombCache = 16;
__global__ void __launch_bounds__(kCombRows * kCombParts) ce_combine_kernel(
    const float* __restrict__ pm, const float* __restrict__ ps, const float* __restrict__ ylab,
    const int32_t* __restrict__ labels, int M, int N, int nblk, float* __restrict__ loss,
    float* __restrict__ lse_out) {
  __shared__ float red[kCombParts][kCombRows];
  __shared__ int bad[kCombParts][kCombRows];
  const int r = threadIdx.x % kCombRows, q = threadIdx.x / kCombRows;
  const int row = blockIdx.x * kCombRows + r;
  const bool live = row < M;
  float m = -INFINITY;
  int nan_seen = 0;
  float cm[kCombCache], cs[kCombCache];
#pragma unroll
  for (int u = 0; u < kCombCache; ++u) {
    const int t = q + u * kCombParts;
    const bool ok = live && t < nblk;
    const int64_t i = (int64_t)t * M + row;
    cs[u] = ok ? ps[i] : 0.f;
    cm[u] = ok ? pm[i] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < kCombCache; ++u) {
    if (cs[u] > 0.f) m = fmaxf(m, cm[u]);
    else if (cs[u] != cs[u]) nan_seen = 1;
  }
  if (live) {
#pragma unroll 4
    for (int t = q + kCombCache * kCombParts; t < nblk; t += kCombParts) {
      const int64_t i = (int64_t)t * M + row;
      const float st = ps[i], mt = pm[i];
      if (st > 0.f) m = fmaxf(m, mt);
      else if (st != st) nan_seen = 1;
    }
  }
  red[q][r] = m;
  bad[q][r] = nan_seen;
  __syncthreads();
  float mx = red[0][r];
  int any_nan = bad[0][r];
#pragma unroll
  for (int j = 1; j < kCombParts; ++j) {
    mx = fmaxf(mx, red[j][r]);
    any_nan |= bad[j][r];
  }
  __syncthreads();
  float sum = 0.f;
#pragma unroll
  for (int u = 0; u < kCombCache; ++u)
    if (cs[u] > 0.f) sum += cs[u] * exp_f(cm[u] - mx);
  if (live) {
#pragma unroll 4
    for (int t = q + kCombCache * kCombParts; t < nblk; t += kCombParts) {
      const int64_t i = (int64_t)t * M + row;
      const float st = ps[i], mt = pm[i];
      if (st > 0.f) sum += st * exp_f(mt - mx);
    }
  }
  red[q][r] = sum;
  __syncthreads();
  if (q != 0 || !live) return;
  float s = red[0][r];
#pragma unroll
  for (int j = 1; j < kCombParts; ++j) s += red[j][r];
  const float lse = any_nan ? __int_as_float(0x7fc00000) : mx + log2f(s) * kLn2F;
  const int lab = labels[row];
  loss[row] = (lab >= 0 && lab < N) ? lse - ylab[row] : __int_as_float(0x7fc00000);
  lse_out[row] = lse;
}

// grad[r, c] currently holds bf16(exp(y - m_blk)); rescale by
// exp(m_blk - lse) and subtract the one-hot term.  Each thread handles 8
// consecutive columns of one row (one 16-byte vector when aligned).
__global__ void __launch_bounds__(256) ce_grad_fixup_kernel(
    uint16_t* __restrict__ grad, int64_t ldc, const float* __restrict__ pm,
    const float* __restrict__ lse, const int32_t* __restrict__ labels, int M, int N,
    int blk_cols, int vec_ok) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int groups = (N + 7) >> 3;
  const int64_t row64 = gid / groups;
  if (row64 >= M) return;
  const int row = (int)row64;
  const int c0 = (int)(gid - row64 * groups) * 8;
  const float l = lse[row];
  const int lab = labels[row];
  uint16_t* g = grad + row64 * ldc + c0;
  if (vec_ok && c0 + 8 <= N && (c0 / blk_cols) == ((c0 + 7) / blk_cols)) {
    const float scale = exp_f(pm[(int64_t)(c0 / blk_cols) * M + row] - l);
    uint4 v = *reinterpret_cast<const uint4*>(g);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + 2 * q;
      const float lo = ce_grad_value(w[q] & 0xffffu, scale, c == lab);
      const float hi = ce_grad_value(w[q] >> 16, scale, c + 1 == lab);
      w[q] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<uint4*>(g) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    for (int e = 0; e < 8 && c0 + e < N; ++e) {
      const int c = c0 + e;
      const float scale = exp_f(pm[(int64_t)(c / blk_cols) * M + row] - l);
      g[e] = to_bf16(ce_grad_value(g[e], scale, c == lab));
    }
  }
}

// The exported scale table of the deferred gradient: s[c][m] = exp(m_b -
// lse[m]) for every 64-column chunk c of row m (b = the CE block holding the
// chunk: the same value for the chunks of one block), fp32 [nchunk][M].
__global__ void __launch_bounds__(256) ce_scale_kernel(const float* __restrict__ pm,
                                                       const float* __restrict__ lse, int M,
                                                       int nchunk, int chunks_per_blk,
                                                       float* __restrict__ scale) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)nchunk * M) return;
  const int c = (int)(gid / M);
  const int row = (int)(gid - (int64_t)c * M);
  scale[gid] = exp_f(pm[(int64_t)(c / chunks_per_blk) * M + row] - lse[row]);
}

}  // namespace

hipError_t launch_ce_scale(const float* part_m, const float* lse, int M, int N, int blk_cols,
                           float* scale, hipStream_t s) {
  const int nchunk = (N + kCeScaleCols - 1) / kCeScaleCols;
  const int64_t threads = (int64_t)nchunk * M;
  hipLaunchKernelGGL(ce_scale_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     part_m, lse, M, nchunk, blk_cols / kCeScaleCols, scale);
  return hipGetLastError();
}

hipError_t launch_ce_combine(const float* part_m, const float* part_s, const float* ylabel,
                             const int32_t* labels, int M, int N, int nblk, float* loss,
                             float* lse, hipStream_t s) {
  const int blocks = (M + kCombRows - 1) / kCombRows;
  hipLaunchKernelGGL(ce_combine_kernel, dim3(blocks), dim3(kCombRows * kCombParts), 0, s, part_m,
                     part_s, ylabel, labels, M, N, nblk, loss, lse);
  return hipGetLastError();
}

hipError_t launch_ce_grad_fixup(uint16_t* grad, int64_t ldc, const float* part_m,
                                const float* lse, const int32_t* labels, int M, int N,
                                int blk_cols, hipStream_t s) {
  const int groups = (N + 7) / 8;
  const int64_t threads = (int64_t)M * groups;
  const int64_t blocks = (threads + 255) / 256;
  const int vec_ok = ((reinterpret_cast<uintptr_t>(grad) & 15) == 0) && (ldc % 8 == 0);
  hipLaunchKernelGGL(ce_grad_fixup_kernel, dim3((unsigned)blocks), dim3(256), 0, s, grad, ldc,
                     part_m, lse, labels, M, N, blk_cols, vec_ok);
  return hipGetLastError();
}

}  // namespace tgemm
