// Eight-wave "ping-pong" matrix-core GEMM for operands that are both
// K-contiguous (A 'N', B 'T'): the layout of a weight stored [N,K] and read
// in place.  Included by the NT translation unit.
//
// One workgroup = 8 wave64s owns a 256x256 output tile, two waves per SIMD.
// Waves 0-3 (group 0) and 4-7 (group 1) sit on SIMDs 0-3 in the same order,
// so every SIMD holds one wave of each group.  The groups run half a phase
// apart, separated by workgroup barriers:
//
//   phase      group 0                          group 1
//   2k         LDS -> registers for k-step k,   32 MFMAs of k-step k-1
//              global -> LDS copies of k+1
//   2k+1       32 MFMAs of k-step k             LDS -> registers for k-step k
//
// so while one wave of a SIMD issues matrix-core work the other waits on
// memory, and the matrix core of every SIMD stays fed.  Each wave holds the
// operand fragments of a whole k-step (64) in registers and computes a
// 128x64 sub-tile (4x2 blocks of 32x32, fp32 accumulators).  LDS holds two
// stages (k-steps) of both 256x64 panels in the same swizzled image the
// four-wave kernel uses, so results are bitwise identical to it.
//
// Hazards (barrier numbers count the barriers each wave executes):
//  * the copies of k-step k+1 land in the stage group 1 last read in phase
//    2k-1; they are issued in phase 2k;
//  * group 0 waits for its copies at the end of phase 2k+1, before either
//    group reads stage k+1 (phases 2k+2 and 2k+3);
//  * every wave's LDS reads complete before the barrier that ends its
//    memory phase (the barrier's fence waits for them).
#pragma once

#include "gemm_kernel.h"

namespace tgemm {

constexpr int kPPThreads = 512;

template <int EPI>
__global__ void __launch_bounds__(kPPThreads, 1) gemm_pp_kernel(GemmParams p) {
  constexpr int BM = 256, BN = 256, WM = 128, WN = 64, FM = WM / 32, FN = WN / 32;
  constexpr int SA = BM * kBK, SB = BN * kBK, STAGE = SA + SB;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;  // 0..7
  const int grp = wave >> 2;                   // ping-pong group
  const int wm = wave & 1, wn = wave >> 1;     // rows wm*128.., cols wn*64..
  const int h = lane >> 5, lc = lane & 31;

  int tm, tn;
  map_tile(blockIdx.x, p.tilesM, p.tilesN, p.groupM, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int a_base = (wm * WM + lc) * kBK;
  const int b_base = SA + (wn * WN + lc) * kBK;
  int xo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) xo[s] = ((2 * s + h) ^ ((lc >> 1) & 7)) << 3;

  const bool interior = p.aligned && m0 + BM <= p.M && n0 + BN <= p.N && (p.K % kBK) == 0 &&
                        p.lda < (1 << 23) && p.ldb < (1 << 23);
  if (interior) {
    const int nk = p.K / kBK;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int grp_u = wave_u >> 2;
    DmaPanel<BM> da;  // group 0 copies both panels: 8 + 8 blocks of 1 KB per wave
    DmaPanel<BN> db;
    da.init(p.lda, wave & 3, lane);
    db.init(p.ldb, wave & 3, lane);
    const uint16_t* oa = p.A + (int64_t)m0 * p.lda;
    const uint16_t* ob = p.B + (int64_t)n0 * p.ldb;
    if (grp_u == 0) {
      da.issue(oa, lds, wave_u);
      db.issue(ob, lds + SA, wave_u);
      wait_dma();
    }
    __syncthreads();
    if (grp_u == 1) __builtin_amdgcn_s_barrier();  // group 1 starts one phase later

    bf16x8_t fa[4][FM], fb[4][FN];
    for (int kt = 0; kt < nk; ++kt) {
      // ---- memory phase: fragments of k-step kt; copies of kt+1 ----
      const uint16_t* cur = lds + (kt & 1) * STAGE;
      if (grp_u == 0 && kt + 1 < nk) {
        uint16_t* nxt = lds + ((kt & 1) ^ 1) * STAGE;
        const int kn = (kt + 1) * kBK;
#pragma unroll
        for (int j = 0; j < BM / 32; ++j) {
          da.issue_one(oa + kn, nxt, wave_u, j);
          db.issue_one(ob + kn, nxt + SA, wave_u, j);
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) read_frags<FM, FN>(cur, a_base, b_base, xo[s], fa[s], fb[s]);
      // The scheduling fences keep every instruction inside its phase: the
      // compiler may not hoist matrix-core work above the barrier (it does
      // not touch memory, so the barrier alone would not stop it).
      // End of the memory phase: this wave's fragment reads have completed
      // (lgkmcnt), its copies may still be in flight.  A plain s_barrier: the
      // workgroup fence of __syncthreads would also wait for the copies.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // ---- compute phase ----
#pragma unroll
      for (int s = 0; s < 4; ++s) mfma_block<FM, FN>(fa[s], fb[s], acc);
      // End of the compute phase: group 0's copies of k-step kt+1 have
      // landed in LDS before anyone passes this barrier.
      __builtin_amdgcn_sched_barrier(0);
      if (grp_u == 0) wait_dma();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (grp_u == 0) __builtin_amdgcn_s_barrier();  // match group 1's extra barrier
  } else {
    // Edge tiles: register-staged (masked) loads, all eight waves in step.
    typename LoaderSel<true, BM, kPPThreads>::type la;
    typename LoaderSel<true, BN, kPPThreads>::type lb;
    const int nk = (p.K + kBK - 1) / kBK;
    const bool aligned = p.aligned != 0;
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
  __syncthreads();  // LDS free for the epilogue
  epilogue<EPI, FM, FN, BM, kPPThreads>(p, acc, m0, n0, wm * WM, wn * WN, tn * 4 + wn, lds, tid,
                                        lane);
}

inline hipError_t launch_gemm_pp(int epi, const GemmParams& p, hipStream_t s) {
  const dim3 grid(p.tilesM * p.tilesN), block(kPPThreads);
  switch (epi) {
    case kEpiStoreBf16:
      hipLaunchKernelGGL((gemm_pp_kernel<kEpiStoreBf16>), grid, block, 0, s, p);
      break;
    case kEpiStoreF32:
      hipLaunchKernelGGL((gemm_pp_kernel<kEpiStoreF32>), grid, block, 0, s, p);
      break;
    default:
      hipLaunchKernelGGL((gemm_pp_kernel<kEpiCE>), grid, block, 0, s, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace tgemm
