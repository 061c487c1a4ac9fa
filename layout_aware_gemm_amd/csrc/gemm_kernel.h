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

// Physical 16-byte chunk of logical chunk c in LDS row `row` is
// c ^ (row & 7).  Eight consecutive rows reading the same logical chunk hit
// eight distinct chunk positions (bank groups), and so do the writers: the
// K-contiguous loader writes the 8 chunks of one row per 8 lanes, the
// transposing loader writes one row per lane group with the k-chunk varying
// fastest across lanes.  The XOR depends on the row only through row & 7,
// so a lane's fragment addresses differ by immediate offsets across the
// 32-row blocks it reads.
__device__ __forceinline__ int swz(int row) { return row & 7; }

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
// Thread t owns k-group kb = t % KBN (L consecutive k) of mn-chunk
// mc = t / KBN (8 consecutive rows of the panel); it loads L 16-byte vectors
// (one per k) and transposes them.  The k-group varies fastest across lanes
// so the transposed LDS writes of a lane group cover distinct chunks of one
// row, while each global load instruction still covers whole 128-byte lines
// (8 lanes with consecutive mc read 128 contiguous bytes of one k row).
template <int R>
struct LoaderMNMajor {
  static constexpr int L = R / 32;    // k values per thread per k-step
  static constexpr int KBN = kBK / L; // k-groups per k-step
  uint4 v[L];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ X, int64_t ld, int r0,
                                       int Rt, int k0, int K, bool aligned, int tid) {
    const int kb = tid % KBN, mc = tid / KBN;
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
    const int kb = tid % KBN, mc = tid / KBN;
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
// Direct global -> LDS panel copy (interior tiles of K-contiguous operands).
//
// One wave-wide 16-byte load with the LDS destination writes 64 x 16 B =
// 1 KB of LDS = 8 panel rows of 128 B, lane l landing at row l/8, physical
// chunk l%8 of that block.  Each lane therefore fetches the logical chunk
// (l%8) ^ swz(row) of its row, which produces exactly the swizzled image the
// register path writes.  No VGPRs hold the data and no LDS write
// instructions are issued.
// ----------------------------------------------------------------------
template <int R>
struct DmaPanel {
  static constexpr int PER_WAVE = R / 32;  // 1 KB blocks issued by each of the 4 waves
  uint32_t off[PER_WAVE];                  // per-lane byte offsets from the panel origin

  __device__ __forceinline__ void init(int64_t ld, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int row = (wave * PER_WAVE + j) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(row);
      off[j] = (uint32_t)(((int64_t)row * ld + c * 8) * 2);
    }
  }

  // origin = &X[r0][k0] (row r0 of the tile, k-step k0), wave-uniform.
  __device__ __forceinline__ void issue(const uint16_t* origin, uint16_t* panel,
                                        int wave_u) const {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int blk = wave_u * PER_WAVE + j;
#if defined(__HIP_DEVICE_COMPILE__)
      // (device pass only: the host pass cannot form the LDS address-space
      // pointer and would silently drop the kernel's launch stub)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const char*>(origin) + off[j],
          (__attribute__((address_space(3))) void*)(panel + blk * 512), 16, 0, 0);
#else
      (void)origin, (void)panel, (void)blk;
#endif
    }
  }
};

// Wait until every global -> LDS copy this wave issued has landed.
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Operand fragments of k-substep s (k = 16s .. 16s+15) for this wave.
// a_base / b_base: element offset of the lane's first A / B row in a stage;
// xo[s]: swizzled element offset of the lane's 16-byte chunk in substep s.
// Successive 32-row blocks are 32 LDS rows (4 KB) apart: immediate offsets.
template <int FM, int FN>
__device__ __forceinline__ void read_frags(const uint16_t* st, int a_base, int b_base, int xo,
                                           bf16x8_t* af, bf16x8_t* bfr) {
  const uint16_t* pa = st + a_base + xo;
  const uint16_t* pb = st + b_base + xo;
#pragma unroll
  for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * kBK);
#pragma unroll
  for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(pb + j * 32 * kBK);
}

template <int FM, int FN>
__device__ __forceinline__ void mfma_block(const bf16x8_t* af, const bf16x8_t* bfr,
                                           f32x16_t (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
}

// Scheduling pattern of one k-substep region: FM*FN MFMAs, FM+FN fragment
// reads and NDMA global->LDS copies.  One read (and up to two copies) is
// placed after each of the first FM+FN MFMAs; the remaining MFMAs follow.
template <int FM, int FN, int NDMA>
__device__ __forceinline__ void sched_substep() {
  constexpr int NRD = FM + FN, NMF = FM * FN;
  constexpr int DPER = (NDMA + NRD - 1) / NRD;
#pragma unroll
  for (int i = 0; i < NRD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    if constexpr (NDMA > 0) __builtin_amdgcn_sched_group_barrier(0x020, DPER, 0);  // VMEM read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NMF - NRD, 0);
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

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // LDS addressing of this lane's operand fragments (see read_frags).
  const int a_base = (wm * WM + lc) * kBK;
  const int b_base = SA + (wn * WN + lc) * kBK;
  int xo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) xo[s] = ((2 * s + h) ^ (lc & 7)) << 3;

  const bool interior = aligned && m0 + BM <= p.M && n0 + BN <= p.N && (p.K % kBK) == 0 &&
                        p.lda < (1 << 23) && p.ldb < (1 << 23);
  if (A_KMAJOR && B_KMAJOR && interior) {
    // Fast path: global -> LDS copies, one barrier per k-step, operand
    // fragments double-buffered in registers so the LDS reads of the next
    // k-substep overlap the matrix-core work of the current one.  The
    // scheduling barriers pin that interleave: each substep region issues
    // one fragment read (and in substep 0 the next stage's copies) between
    // consecutive MFMAs.
    const int nk = p.K / kBK;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    DmaPanel<BM> da;
    DmaPanel<BN> db;
    da.init(p.lda, wave, lane);
    db.init(p.ldb, wave, lane);
    const uint16_t* oa = p.A + (int64_t)m0 * p.lda;
    const uint16_t* ob = p.B + (int64_t)n0 * p.ldb;
    da.issue(oa, lds, wave_u);
    db.issue(ob, lds + SA, wave_u);
    wait_dma();
    __syncthreads();
    bf16x8_t fa[2][FM], fb[2][FN];
    read_frags<FM, FN>(lds, a_base, b_base, xo[0], fa[0], fb[0]);
    for (int kt = 0; kt < nk; ++kt) {
      const uint16_t* cur = lds + (kt & 1) * STAGE;
      uint16_t* nxt = lds + ((kt & 1) ^ 1) * STAGE;
      // substep 0 (+ next stage's copies; in the last iteration the copy
      // re-reads the first k-step into the idle stage, unused)
      const int kn = (kt + 1 < nk) ? (kt + 1) * kBK : 0;
      da.issue(oa + kn, nxt, wave_u);
      db.issue(ob + kn, nxt + SA, wave_u);
      read_frags<FM, FN>(cur, a_base, b_base, xo[1], fa[1], fb[1]);
      mfma_block<FM, FN>(fa[0], fb[0], acc);
      sched_substep<FM, FN, (BM + BN) / 32>();
      __builtin_amdgcn_sched_barrier(0);
      // substep 1
      read_frags<FM, FN>(cur, a_base, b_base, xo[2], fa[0], fb[0]);
      mfma_block<FM, FN>(fa[1], fb[1], acc);
      sched_substep<FM, FN, 0>();
      __builtin_amdgcn_sched_barrier(0);
      // substep 2
      read_frags<FM, FN>(cur, a_base, b_base, xo[3], fa[1], fb[1]);
      mfma_block<FM, FN>(fa[0], fb[0], acc);
      sched_substep<FM, FN, 0>();
      __builtin_amdgcn_sched_barrier(0);
      // substep 3: every fragment of this stage is in registers.  The next
      // stage's copies must have landed (own wave: vmcnt; other waves: the
      // barrier) before it is read, and after the barrier the current stage
      // may be overwritten by the next iteration's copies.
      wait_dma();
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      read_frags<FM, FN>(nxt, a_base, b_base, xo[0], fa[0], fb[0]);
      mfma_block<FM, FN>(fa[1], fb[1], acc);
      sched_substep<FM, FN, 0>();
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // General path: any layout, ragged edges, unaligned operands.  16-byte
    // (or masked element) loads into registers, one k-step ahead, then
    // (transposing if needed) stores into the other LDS stage.
    typename LoaderSel<A_KMAJOR, BM>::type la;
    typename LoaderSel<B_KMAJOR, BN>::type lb;
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
        read_frags<FM, FN>(st, a_base, b_base, xo[s], af, bfr);
        mfma_block<FM, FN>(af, bfr, acc);
      }
      if (more) {
        uint16_t* nx = lds + (cur ^ 1) * STAGE;
        la.store(nx, tid);
        lb.store(nx + SA, tid);
      }
      __syncthreads();
    }
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
