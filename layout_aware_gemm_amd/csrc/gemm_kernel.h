// Matrix-core (MFMA) bf16 GEMM for gfx950 with layout flags and fused
// epilogues.  Included by one translation unit per operand layout.
//
// Structure of one workgroup (256 threads = 4 wave64s in a 2x2 grid):
//   * it owns a BM x BN output tile and walks K in steps of 64;
//   * each k-step, every thread fetches its share of the A and B panels
//     with 16-byte global loads along the operand's contiguous axis into
//     registers (the next step's loads are in flight while the current step
//     computes), then writes them to the other half of a double-buffered
//     LDS tile;
//   * LDS always holds both panels K-contiguous ([rows][64] bf16, 128 B per
//     row) with the 16-byte chunks XOR-swizzled, so the matrix-core operand
//     reads below are identical for every layout.  An operand that is
//     contiguous along M or N (A 'T', B 'N') is transposed in registers
//     (8x8 / 4x8 blocks of bf16) on its way into LDS;
//   * each wave multiplies its (BM/2) x (BN/2) sub-tile with
//     v_mfma_f32_32x32x16_bf16, fp32 accumulation in registers.
//
// Because the LDS image and the instruction stream after it do not depend
// on the layout, the four layouts produce bitwise-identical results.
#pragma once

#include "tgemm_internal.h"

namespace tgemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBK = 64;          // k elements per LDS row
constexpr float kLog2e = 1.4426950408889634f;

// Physical 16-byte chunk of logical chunk c in LDS row `row`: XOR with a
// 3-bit hash of the row, chosen so that (a) 8 consecutive rows reading the
// same logical chunk and (b) rows 8 apart (the transposing writer's
// pattern) both land in 8 distinct chunk positions.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ uint32_t u4comp(const uint4& v, int d) {
  return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w;
}

// fp32 -> bf16 bits, round to nearest even, NaN kept quiet.
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ----------------------------------------------------------------------
// Operand loaders.  R = rows of the panel (M or N extent of the tile).
// ----------------------------------------------------------------------

// Operand contiguous along K: stored row r (an m or n index) holds k.
template <int R>
struct LoaderKMajor {
  static constexpr int L = R / 32;  // 16-byte chunks per thread per k-step
  uint4 v[L];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ X, int64_t ld, int r0,
                                       int Rt, int k0, int K, bool aligned, int tid) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int q = tid + kThreads * i;
      const int row = q >> 3, kc = q & 7;
      const int gr = r0 + row, gk = k0 + kc * 8;
      if (aligned && gr < Rt && gk + 8 <= K) {
        v[i] = *reinterpret_cast<const uint4*>(X + (int64_t)gr * ld + gk);
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (gr < Rt) {
          const uint16_t* p = X + (int64_t)gr * ld;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gk + e < K) w[e >> 1] |= (uint32_t)p[gk + e] << ((e & 1) * 16);
        }
        v[i] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int q = tid + kThreads * i;
      const int row = q >> 3, kc = q & 7;
      *reinterpret_cast<uint4*>(lds + row * kBK + ((kc ^ swz(row)) << 3)) = v[i];
    }
  }
};

// Operand contiguous along M/N: stored row k holds the m (or n) index.
// Thread t owns mn-chunk (t % CPR) (8 consecutive rows of the panel) and
// L consecutive k; it loads L 16-byte vectors and transposes them.
template <int R>
struct LoaderMNMajor {
  static constexpr int L = R / 32;   // k values per thread per k-step
  static constexpr int CPR = R / 8;  // 8-wide mn chunks per stored k row
  uint4 v[L];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ X, int64_t ld, int r0,
                                       int Rt, int k0, int K, bool aligned, int tid) {
    const int mc = tid % CPR, kb = tid / CPR;
    const int gr = r0 + mc * 8;
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int gk = k0 + kb * L + j;
      if (aligned && gk < K && gr + 8 <= Rt) {
        v[j] = *reinterpret_cast<const uint4*>(X + (int64_t)gk * ld + gr);
      } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (gk < K) {
          const uint16_t* p = X + (int64_t)gk * ld;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (gr + e < Rt) w[e >> 1] |= (uint32_t)p[gr + e] << ((e & 1) * 16);
        }
        v[j] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }

  __device__ __forceinline__ uint32_t elem(int j, int i) const {
    return (u4comp(v[j], i >> 1) >> ((i & 1) * 16)) & 0xffffu;
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
    const int mc = tid % CPR, kb = tid / CPR;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = mc * 8 + i;
      uint16_t* dst = lds + row * kBK;
      if constexpr (L == 8) {
        uint4 o;
        o.x = elem(0, i) | (elem(1, i) << 16);
        o.y = elem(2, i) | (elem(3, i) << 16);
        o.z = elem(4, i) | (elem(5, i) << 16);
        o.w = elem(6, i) | (elem(7, i) << 16);
        *reinterpret_cast<uint4*>(dst + ((kb ^ swz(row)) << 3)) = o;
      } else if constexpr (L == 4) {
        uint2 o;
        o.x = elem(0, i) | (elem(1, i) << 16);
        o.y = elem(2, i) | (elem(3, i) << 16);
        *reinterpret_cast<uint2*>(dst + (((kb >> 1) ^ swz(row)) << 3) + (kb & 1) * 4) = o;
      } else {
        static_assert(L == 2, "panel rows must be 64, 128 or 256");
        const uint32_t o = elem(0, i) | (elem(1, i) << 16);
        *reinterpret_cast<uint32_t*>(dst + (((kb >> 2) ^ swz(row)) << 3) + (kb & 3) * 2) = o;
      }
    }
  }
};

template <bool KMAJOR, int R>
struct LoaderSel {
  using type = LoaderKMajor<R>;
};
template <int R>
struct LoaderSel<false, R> {
  using type = LoaderMNMajor<R>;
};

// ----------------------------------------------------------------------
// Workgroup -> tile mapping.  Workgroups are dealt round-robin to the 8
// XCDs (workgroup b runs on XCD b % 8), each with its own L2.  The first
// 8*floor(T/8) workgroups are renumbered so XCD x gets a contiguous range
// of logical tiles; logical tiles are then ordered in groups of `groupM`
// tile rows (column-major inside a group), so the tiles one XCD runs at
// the same time share A rows and B columns in its L2.
// ----------------------------------------------------------------------
__device__ __forceinline__ void map_tile(int bid, int tilesM, int tilesN, int groupM, int& tm,
                                         int& tn) {
  const int T = tilesM * tilesN;
  const int per = T >> 3;
  int l = bid;
  if (bid < per * 8) l = (bid & 7) * per + (bid >> 3);
  const int gsz = groupM * tilesN;
  const int g = l / gsz, r = l - g * gsz;
  const int gm0 = g * groupM;
  const int gm = min(groupM, tilesM - gm0);
  tm = gm0 + r % gm;
  tn = r / gm;
}

template <int N>
__device__ __forceinline__ float xor_max(float v) {
#pragma unroll
  for (int o = 1; o < N; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
template <int N>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
  for (int o = 1; o < N; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ----------------------------------------------------------------------
// The kernel.
// ----------------------------------------------------------------------
template <int BM, int BN, bool A_KMAJOR, bool B_KMAJOR, int EPI>
__global__ void __launch_bounds__(kThreads, 1) gemm_kernel(GemmParams p) {
  constexpr int WM = BM / 2, WN = BN / 2;   // wave sub-tile
  constexpr int FM = WM / 32, FN = WN / 32; // 32x32 blocks per wave
  constexpr int SA = BM * kBK, SB = BN * kBK, STAGE = SA + SB;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, lc = lane & 31;

  int tm, tn;
  map_tile(blockIdx.x, p.tilesM, p.tilesN, p.groupM, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const bool aligned = p.aligned != 0;

  typename LoaderSel<A_KMAJOR, BM>::type la;
  typename LoaderSel<B_KMAJOR, BN>::type lb;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // LDS offsets of this lane's operand rows.
  int arow[FM], asw[FM], brow[FN], bsw[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int r = wm * WM + i * 32 + lc;
    arow[i] = r * kBK;
    asw[i] = swz(r);
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int r = wn * WN + j * 32 + lc;
    brow[j] = SA + r * kBK;
    bsw[j] = swz(r);
  }

  const int nk = (p.K + kBK - 1) / kBK;
  la.load(p.A, p.lda, m0, p.M, 0, p.K, aligned, tid);
  lb.load(p.B, p.ldb, n0, p.N, 0, p.K, aligned, tid);
  la.store(lds, tid);
  lb.store(lds + SA, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(p.A, p.lda, m0, p.M, (kt + 1) * kBK, p.K, aligned, tid);
      lb.load(p.B, p.ldb, n0, p.N, (kt + 1) * kBK, p.K, aligned, tid);
    }
    const uint16_t* st = lds + cur * STAGE;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t af[FM], bfr[FN];
      const int c = 2 * s + h;  // logical 16-byte chunk: k = 16s + 8h .. +7
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(st + arow[i] + ((c ^ asw[i]) << 3));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(st + brow[j] + ((c ^ bsw[j]) << 3));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      uint16_t* nx = lds + (cur ^ 1) * STAGE;
      la.store(nx, tid);
      lb.store(nx + SA, tid);
    }
    __syncthreads();
  }

  // Accumulator layout of v_mfma_f32_32x32x16: lane l, register r holds
  // row 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the 32x32 block.
  if constexpr (EPI == kEpiStoreBf16 || EPI == kEpiStoreF32) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * WN + j * 32 + lc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row < p.M && col < p.N) {
            if constexpr (EPI == kEpiStoreBf16)
              reinterpret_cast<uint16_t*>(p.C)[(int64_t)row * p.ldc + col] =
                  (uint16_t)f2bf(acc[i][j][r]);
            else
              reinterpret_cast<float*>(p.C)[(int64_t)row * p.ldc + col] = acc[i][j][r];
          }
        }
      }
  } else {
    // Cross-entropy epilogue.  Per row of this wave's WN-column block:
    // block max, block sum of exp(y - max), the label logit if the label
    // column falls in the block, and optionally exp(y - block max) into
    // the gradient buffer.  The logits themselves are not stored.
    int* slab = reinterpret_cast<int*>(lds);
    for (int t = tid; t < BM; t += kThreads) {
      const int row = m0 + t;
      slab[t] = row < p.M ? p.labels[row] : -1;
    }
    __syncthreads();
    const int pcol = tn * 2 + wn;
    const int64_t pbase = (int64_t)pcol * p.M;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lrow = wm * WM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int row = m0 + lrow;
        const int lab = slab[lrow];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn * WN + j * 32 + lc;
          if (col < p.N) mx = fmaxf(mx, acc[i][j][r]);
        }
        mx = xor_max<32>(mx);
        float sum = 0.f, ylab = 0.f;
        bool hit = false;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn * WN + j * 32 + lc;
          const float y = acc[i][j][r];
          const float e = exp2f((y - mx) * kLog2e);
          const bool ok = col < p.N;
          sum += ok ? e : 0.f;
          hit = hit || (col == lab);
          ylab = (col == lab) ? y : ylab;
          if (p.grad && ok && row < p.M) p.grad[(int64_t)row * p.ldc + col] = (uint16_t)f2bf(e);
        }
        if (hit && row < p.M) p.ylabel[row] = ylab;
        sum = xor_sum<32>(sum);
        if (lc == r && row < p.M) {
          p.part_m[pbase + row] = mx;
          p.part_s[pbase + row] = sum;
        }
      }
    }
  }
}

// Host-side launch of one instantiation.
template <int BM, int BN, bool AK, bool BK>
hipError_t launch_gemm_tpl(int epi, const GemmParams& p, hipStream_t s) {
  const dim3 grid(p.tilesM * p.tilesN), block(kThreads);
  switch (epi) {
    case kEpiStoreBf16:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BK, kEpiStoreBf16>), grid, block, 0, s, p);
      break;
    case kEpiStoreF32:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BK, kEpiStoreF32>), grid, block, 0, s, p);
      break;
    default:
      hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BK, kEpiCE>), grid, block, 0, s, p);
      break;
  }
  return hipGetLastError();
}

template <bool AK, bool BK>
hipError_t launch_gemm_layout(int cfg, int epi, const GemmParams& p, hipStream_t s) {
  if (cfg == kTile256) return launch_gemm_tpl<256, 256, AK, BK>(epi, p, s);
  return launch_gemm_tpl<128, 128, AK, BK>(epi, p, s);
}

}  // namespace tgemm
