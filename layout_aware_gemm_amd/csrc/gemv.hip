// Matrix-vector products and dot products: a GEMM with M = 1 or N = 1 (and
// K > 1).  "Schedule a small matmul op as a reduction (or pointwise) op"
// (the discussion) weighs decomposing such matmuls -- a 1-D operand (gemv)
// and very long dot products, K of order 10^5 to 10^8 -- instead of running
// them as matmuls.  Here they never touch the matrix cores: every output is
// a K-long reduction that reads each matrix element once, so the kernels
// are bound by HBM bandwidth.
//
// The matrix operand X holds L output rows of K elements each (L = M for
// N = 1, L = N for M = 1; a dot product is L = 1); the other operand is a
// K-vector v.  Two kernel shapes cover the two ways X can be stored:
//   - rowdot: each row of X is K-contiguous (A 'N' for N = 1, B 'T' for
//     M = 1): one wave per (row, K chunk), 16-byte loads of X and v.
//   - colsweep: X is stored [K][L], L-contiguous (A 'T', B 'N'): a
//     workgroup takes 512 consecutive outputs (8 per lane) and splits a K
//     chunk among its four waves; the element v[k] is the same for a wave.
// Both write one fp32 partial per (K chunk, output) to the workspace;
// combine then adds the chunks of each output in a fixed order -- so
// results do not depend on scheduling -- and stores bf16 (round to nearest
// even) or fp32.  With a single chunk the reduction kernel stores the
// output itself and no combine pass runs.
#include "bf16_cvt.h"
#include "tgemm_internal.h"

namespace tgemm {

namespace {

__device__ __forceinline__ void store_out(void* C, int64_t off, float s, int out_f32) {
  if (out_f32) static_cast<float*>(C)[off] = s;
  else static_cast<uint16_t*>(C)[off] = to_bf16(s);
}

// partial[kc * L + r] = sum over k in chunk kc of X[r*ldx + k*sx] * v[k*sv]
// (with a single chunk the sum goes straight to the output C + r*sc).
// Workgroup = 4 waves = 4 (row, chunk) items.  VEC: sx == sv == 1, rows and
// v 16-byte aligned; lanes then take 8 consecutive k per step.
template <bool VEC>
__global__ void __launch_bounds__(256) rowdot_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                     int64_t sx, const uint16_t* __restrict__ v,
                                                     int64_t sv, int L, int64_t K,
                                                     int64_t kchunk, int nkc,
                                                     float* __restrict__ partial, void* C,
                                                     int64_t sc, int out_f32) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)L * nkc) return;
  const int r = (int)(item % L);
  const int kc = (int)(item / L);
  const int64_t k0 = (int64_t)kc * kchunk;
  const int64_t k1 = k0 + kchunk < K ? k0 + kchunk : K;
  const uint16_t* x = X + (int64_t)r * ldx;
  float acc = 0.f;
  int64_t k = k0;
  if constexpr (VEC) {
    // 512 k per wave step; two steps in flight per iteration
    for (; k + 1024 <= k1; k += 1024) {
      const uint4 xa = *reinterpret_cast<const uint4*>(x + k + lane * 8);
      const uint4 va = *reinterpret_cast<const uint4*>(v + k + lane * 8);
      const uint4 xb = *reinterpret_cast<const uint4*>(x + k + 512 + lane * 8);
      const uint4 vb = *reinterpret_cast<const uint4*>(v + k + 512 + lane * 8);
      const uint32_t xw[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
      const uint32_t vw[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        acc = fmaf(from_bf16(xw[q] & 0xffffu), from_bf16(vw[q] & 0xffffu), acc);
        acc = fmaf(from_bf16(xw[q] >> 16), from_bf16(vw[q] >> 16), acc);
      }
    }
    for (; k + 512 <= k1; k += 512) {
      const uint4 xa = *reinterpret_cast<const uint4*>(x + k + lane * 8);
      const uint4 va = *reinterpret_cast<const uint4*>(v + k + lane * 8);
      const uint32_t xw[4] = {xa.x, xa.y, xa.z, xa.w};
      const uint32_t vw[4] = {va.x, va.y, va.z, va.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc = fmaf(from_bf16(xw[q] & 0xffffu), from_bf16(vw[q] & 0xffffu), acc);
        acc = fmaf(from_bf16(xw[q] >> 16), from_bf16(vw[q] >> 16), acc);
      }
    }
  }
  // remaining k (or all of them without VEC), one element per lane per step
  for (k += lane; k < k1; k += 64)
    acc = fmaf(from_bf16(x[k * sx]), from_bf16(v[k * sv]), acc);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane != 0) return;
  if (nkc > 1) partial[(int64_t)kc * L + r] = acc;
  else store_out(C, (int64_t)r * sc, acc, out_f32);  // one chunk: no combine pass
}

// partial[kc * L + c] = sum over k in chunk kc of X[k*ldx + c] * v[k*sv].
// A workgroup takes 512 consecutive c (8 per lane) and the chunk's rows in
// four consecutive quarters, one per wave; the four wave sums are then
// added in wave order through LDS.  Four waves per 512 outputs, rather than
// one wave per 512 outputs and four times as many chunks, keep enough
// loads in flight without four times the partials.  VEC: ldx % 8 == 0 and
// X 16-byte aligned.
constexpr int kSweepCols = 512;

template <bool VEC>
__global__ void __launch_bounds__(256) colsweep_kernel(const uint16_t* __restrict__ X,
                                                       int64_t ldx, const uint16_t* __restrict__ v,
                                                       int64_t sv, int L, int64_t K,
                                                       int64_t kchunk, int nkc,
                                                       float* __restrict__ partial, void* C,
                                                       int64_t sc, int out_f32) {
  __shared__ float red[4][kSweepCols];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c0 = blockIdx.x * kSweepCols + lane * 8;
  const int kc = blockIdx.y;
  const int64_t k0 = (int64_t)kc * kchunk;
  const int64_t k1 = k0 + kchunk < K ? k0 + kchunk : K;
  const int64_t qr = (k1 - k0 + 3) / 4;  // rows per wave
  const int64_t kw0 = k0 + wave * qr < k1 ? k0 + wave * qr : k1;
  const int64_t kw1 = kw0 + qr < k1 ? kw0 + qr : k1;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c0 < L) {
    if (VEC && c0 + 8 <= L) {
      int64_t k = kw0;
      for (; k + 4 <= kw1; k += 4) {
        uint4 xr[4];
        float vk[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          xr[u] = *reinterpret_cast<const uint4*>(X + (k + u) * ldx + c0);
          vk[u] = from_bf16(v[(k + u) * sv]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t w[4] = {xr[u].x, xr[u].y, xr[u].z, xr[u].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] = fmaf(from_bf16(w[q] & 0xffffu), vk[u], acc[2 * q]);
            acc[2 * q + 1] = fmaf(from_bf16(w[q] >> 16), vk[u], acc[2 * q + 1]);
          }
        }
      }
      for (; k < kw1; ++k) {
        const uint4 xr = *reinterpret_cast<const uint4*>(X + k * ldx + c0);
        const float vk = from_bf16(v[k * sv]);
        const uint32_t w[4] = {xr.x, xr.y, xr.z, xr.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(from_bf16(w[q] & 0xffffu), vk, acc[2 * q]);
          acc[2 * q + 1] = fmaf(from_bf16(w[q] >> 16), vk, acc[2 * q + 1]);
        }
      }
    } else {
      for (int64_t k = kw0; k < kw1; ++k) {
        const float vk = from_bf16(v[k * sv]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + e < L) acc[e] = fmaf(from_bf16(X[k * ldx + c0 + e]), vk, acc[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[wave][lane * 8 + e] = acc[e];
  __syncthreads();
  if (wave != 0 || c0 >= L) return;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (c0 + e >= L) continue;
    const int i = lane * 8 + e;
    const float t = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
    if (nkc > 1) partial[(int64_t)kc * L + c0 + e] = t;
    else store_out(C, (int64_t)(c0 + e) * sc, t, out_f32);
  }
}

// y[r] = sum over kc = 0, 1, ..., nkc-1 of partial[kc * L + r], stored at
// C + r*sc, in one of three fixed orders (each deterministic):
//   MODE 0 (few chunks): one thread per output adds the chunks in order.
//   MODE 1 (many chunks, many outputs): a workgroup takes 16 consecutive
//     outputs and 16 chunk lanes; lane q adds chunks q, q+16, q+32, ...
//     (the 16 threads of a lane read 16 consecutive partials), then the 16
//     lane sums are added in ascending q.
//   MODE 2 (many chunks, under 16 outputs): a workgroup per output; thread t
//     adds chunks t, t+256, ..., then the 256 sums are folded pairwise in a
//     fixed tree.
// 0 + partial[kc*L + r] + ... for kc = kc0, kc0 + step, ... < nkc, added in
// that order.  Eight loads are issued before the first addition waits, so a
// thread waits for memory once per eight chunks, not once per chunk.
__device__ __forceinline__ float add_strided(const float* __restrict__ partial, int L, int64_t r,
                                             int kc0, int step, int nkc) {
  float t = 0.f;
  for (int base = kc0; base < nkc; base += 8 * step) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kc = base + u * step;
      v[u] = kc < nkc ? partial[(int64_t)kc * L + r] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (base + u * step < nkc) t += v[u];
  }
  return t;
}

template <int MODE>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ partial, int L,
                                                      int nkc, void* __restrict__ C, int64_t sc,
                                                      int out_f32) {
  float s;
  int64_t r;
  if constexpr (MODE == 2) {
    __shared__ float red[256];
    r = blockIdx.x;
    float t = 0.f;
    t = add_strided(partial, L, r, (int)threadIdx.x, 256, nkc);
    red[threadIdx.x] = t;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x != 0) return;
    s = red[0];
  } else if constexpr (MODE == 1) {
    __shared__ float red[16][16];
    const int j = threadIdx.x & 15, q = threadIdx.x >> 4;
    r = (int64_t)blockIdx.x * 16 + j;
    float t = 0.f;
    if (r < L) t = add_strided(partial, L, r, q, 16, nkc);
    red[q][j] = t;
    __syncthreads();
    if (q != 0 || r >= L) return;
    s = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) s += red[u][j];
  } else {
    r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (r >= L) return;
    s = 0.f;
    s = add_strided(partial, L, r, 0, 1, nkc);
  }
  store_out(C, r * sc, s, out_f32);
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int64_t gemv_chunks(int shape, int L, int64_t K) {
  if (shape == kGemvRows) {
    // at least ~4096 waves, chunks of at least 4096 elements
    int64_t n = cdiv(4096, L);
    const int64_t most = cdiv(K, 4096);
    if (n > most) n = most;
    return n < 1 ? 1 : n;
  }
  // colsweep: at least ~2048 workgroups of 512 outputs, chunks of at least
  // 64 rows (16 per wave)
  const int64_t cb = cdiv(L, 512);
  int64_t n = cdiv(2048, cb);
  const int64_t most = cdiv(K, 64);
  if (n > most) n = most;
  return n < 1 ? 1 : n;
}

hipError_t launch_gemv(int shape, const uint16_t* X, int64_t ldx, int64_t sx, const uint16_t* v,
                       int64_t sv, int L, int64_t K, int nkc, float* partial, void* C,
                       int64_t sc, bool out_f32, hipStream_t s) {
  if (shape == kGemvRows) {
    int64_t kchunk = cdiv(K, nkc);
    const bool vec = sx == 1 && sv == 1 && (ldx % 8 == 0 || L == 1) &&
                     ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(v)) & 15) == 0;
    if (vec) kchunk = cdiv(kchunk, 512) * 512;  // chunk starts stay 16-byte aligned
    nkc = (int)cdiv(K, kchunk);
    const int64_t items = (int64_t)L * nkc;
    const dim3 grid((unsigned)cdiv(items, 4));
    if (vec)
      hipLaunchKernelGGL(rowdot_kernel<true>, grid, dim3(256), 0, s, X, ldx, sx, v, sv, L, K,
                         kchunk, nkc, partial, C, sc, out_f32 ? 1 : 0);
    else
      hipLaunchKernelGGL(rowdot_kernel<false>, grid, dim3(256), 0, s, X, ldx, sx, v, sv, L, K,
                         kchunk, nkc, partial, C, sc, out_f32 ? 1 : 0);
  } else {
    const int64_t kchunk = cdiv(K, nkc);
    nkc = (int)cdiv(K, kchunk);
    const bool vec = ldx % 8 == 0 && (reinterpret_cast<uintptr_t>(X) & 15) == 0;
    const dim3 grid((unsigned)cdiv(L, kSweepCols), (unsigned)nkc);
    if (vec)
      hipLaunchKernelGGL(colsweep_kernel<true>, grid, dim3(256), 0, s, X, ldx, v, sv, L, K, kchunk,
                         nkc, partial, C, sc, out_f32 ? 1 : 0);
    else
      hipLaunchKernelGGL(colsweep_kernel<false>, grid, dim3(256), 0, s, X, ldx, v, sv, L, K,
                         kchunk, nkc, partial, C, sc, out_f32 ? 1 : 0);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nkc == 1) return e;
  const int of = out_f32 ? 1 : 0;
  if (nkc <= 16)
    hipLaunchKernelGGL(combine_kernel<0>, dim3((unsigned)cdiv(L, 256)), dim3(256), 0, s, partial,
                       L, nkc, C, sc, of);
  else if (L >= 16)
    hipLaunchKernelGGL(combine_kernel<1>, dim3((unsigned)cdiv(L, 16)), dim3(256), 0, s, partial, L,
                       nkc, C, sc, of);
  else
    hipLaunchKernelGGL(combine_kernel<2>, dim3((unsigned)L), dim3(256), 0, s, partial, L, nkc, C,
                       sc, of);
  return hipGetLastError();
}

}  // namespace tgemm
