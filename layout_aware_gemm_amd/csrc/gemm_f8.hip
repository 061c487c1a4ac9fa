// fp8 (e4m3fn) GEMM on gfx950's fp8 matrix cores ("Improve the Inductor
// generated kernel for the pattern of output1 = pointwise(input); output2 =
// transpose(output1)", the example's float8 linear).
//
// Operands: two K-contiguous byte matrices of e4m3fn codes, A8 [Mp][Kp]
// and B8 [Np][Kp], that the pack pass (fp8_cast.hip) wrote from the caller's
// bf16 operands in whatever layout those had, zero-padded to whole tiles
// (Mp, Np multiples of the tile size, Kp of 128).  So every tile is
// interior and both panels reach LDS with the direct global -> LDS copies
// of the bf16 kernel: a byte row of 128 codes is one 128-byte LDS row, the
// same image, swizzle and copy count as a 64-element bf16 k-step.
//
// Each k-step (128 codes) is two substeps of v_mfma_f32_32x32x64_f8f6f4 (fp8
// e4m3 times fp8 e4m3, fp32 accumulation): a lane feeds 32 codes of its row
// (A) or column (B) per MFMA, two 16-byte chunks of the LDS row.  A and B
// lanes take the same chunks in the same order, so whatever order the
// instruction gives the 64 k inside it, it pairs A's code k with B's code k.
// Per k-step the matrix core does the same cycles as the bf16 loop's 64-k
// step (half the MFMAs, each twice as long) for twice the k.
//
// The main loop is the bf16 kernel's three-buffer schedule (two A panels,
// three B panels, 160 KB for 256x256 tiles): the copies of B(kt+2) ride in
// the first substep of kt, one barrier, then the copies of A(kt+2).
#include "gemm_kernel.h"
#include "tgemm_internal.h"

namespace tgemm {
namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// One 32x32x64 MFMA on e4m3fn codes (format 0 for both operands; the zero
// scale operands select the unscaled instruction).  Accumulator layout as
// for the bf16 32x32x16: column = lane % 32, rows across registers.
__device__ __forceinline__ f32x16_t mma_f8(const i32x4_t& a0, const i32x4_t& a1,
                                           const i32x4_t& b0, const i32x4_t& b1,
                                           const f32x16_t& c) {
  const i32x8_t a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
  const i32x8_t b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The operand fragments of one 64-k substep: half h of fragment f is the
// 16-byte chunk h of the lane's row in 32-row block f.
template <int FM, int FN>
struct Frag8 {
  i32x4_t a[FM][2], b[FN][2];
};

// One 64-k substep: MFMA q with `cur`; the half-fragment reads of the next
// substep (chunks at element offsets x0, x1 of the rows at pa / pb) into
// `nxt`; and, when `cp` is set, this wave's copies of one panel (d, origin
// o, into dst).  Item i of n side items goes with slot floor(i * SL / n),
// so they spread evenly over the slots whatever their count.
template <int FM, int FN, int R>
__device__ __forceinline__ void f8_substep(f32x16_t (&acc)[FM][FN], const Frag8<FM, FN>& cur,
                                           Frag8<FM, FN>& nxt, const uint16_t* pa,
                                           const uint16_t* pb, int x0, int x1, bool cp,
                                           const DmaPanel<R>& d, const uint16_t* o,
                                           uint16_t* dst, int wave_u) {
  constexpr int SL = FM * FN, RD = 2 * (FM + FN);
  constexpr int NCP = DmaPanel<R>::PER_WAVE;
#pragma unroll
  for (int q = 0; q < SL; ++q) {
    const int i = q / FN, j = q % FN;
    acc[i][j] = mma_f8(cur.a[i][0], cur.a[i][1], cur.b[j][0], cur.b[j][1], acc[i][j]);
#pragma unroll
    for (int r = 0; r < RD; ++r) {
      if ((r * SL) / RD != q) continue;
      const int f = r >> 1, hf = r & 1;
      const int x = hf ? x1 : x0;
      if (f < FM)
        nxt.a[f][hf] = *reinterpret_cast<const i32x4_t*>(pa + f * 32 * kBK + x);
      else
        nxt.b[f - FM][hf] = *reinterpret_cast<const i32x4_t*>(pb + (f - FM) * 32 * kBK + x);
    }
    if (cp) {
#pragma unroll
      for (int c = 0; c < NCP; ++c)
        if ((c * SL) / NCP == q) d.issue_one(o, dst, wave_u, c);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// nk k-steps of 128 codes.  a_base / b_local: element offsets of the lane's
// first A / B fragment row inside a panel buffer; xo[c]: swizzled element
// offset of the lane's chunk in the bf16 substep c (substep s of this loop
// reads the chunks of bf16 substeps 2s and 2s + 1).
template <int BM, int BN, int FM, int FN>
__device__ __forceinline__ void f8_mainloop(const GemmParams& p, int m0, int n0, int nk,
                                            uint16_t* lds, int wave, int lane, int a_base,
                                            int b_local, const int* xo,
                                            f32x16_t (&acc)[FM][FN]) {
  constexpr int SA = BM * kBK, SB = BN * kBK;
  constexpr int NA = DmaPanel<BM>::PER_WAVE, NB = DmaPanel<BN>::PER_WAVE;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  DmaPanel<BM> da;
  DmaPanel<BN> db;
  da.init(p.lda, wave, lane);
  db.init(p.ldb, wave, lane);
  const uint16_t* oa = p.A + (int64_t)m0 * p.lda;
  const uint16_t* ob = p.B + (int64_t)n0 * p.ldb;
  uint16_t* const abuf = lds;           // two A panels
  uint16_t* const bbuf = lds + 2 * SA;  // three B panels
  // k-steps past the end re-read k-step 0 into a buffer that is never
  // multiplied, which keeps the copy counts, and so the waits, uniform
  auto kof = [nk](int t) { return (t < nk ? t : 0) * kBK; };
  da.issue(oa + kof(0), abuf, wave_u);
  db.issue(ob + kof(0), bbuf, wave_u);
  db.issue(ob + kof(1), bbuf + SB, wave_u);
  da.issue(oa + kof(1), abuf + SA, wave_u);
  // A(0), B(0) landed (own copies; other waves: the barrier)
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(NA + NB, 0));
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  Frag8<FM, FN> F[2];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      F[0].a[i][hf] = *reinterpret_cast<const i32x4_t*>(abuf + a_base + i * 32 * kBK + xo[hf]);
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      F[0].b[j][hf] =
          *reinterpret_cast<const i32x4_t*>(bbuf + b_local + j * 32 * kBK + xo[hf]);
  int b3 = 0;  // kt % 3
  for (int kt = 0; kt < nk; ++kt) {
    const int b3n = b3 == 2 ? 0 : b3 + 1;  // (kt + 1) % 3
    const int b3p = b3 == 0 ? 2 : b3 - 1;  // (kt + 2) % 3, the buffer k-step kt-1 used
    const uint16_t* ac = abuf + (kt & 1) * SA + a_base;
    const uint16_t* bc = bbuf + b3 * SB + b_local;
    const uint16_t* an = abuf + ((kt + 1) & 1) * SA + a_base;
    const uint16_t* bn = bbuf + b3n * SB + b_local;
    __builtin_amdgcn_sched_barrier(0);
    f8_substep<FM, FN, BN>(acc, F[0], F[1], ac, bc, xo[2], xo[3], true, db, ob + kof(kt + 2),
                           bbuf + b3p * SB, wave_u);
    // A(kt+1), B(kt+1) landed (own copies: all but the NB just issued;
    // other waves: the barrier) and this wave's reads of A(kt) are done, so
    // after the barrier A(kt)'s buffer is free for A(kt+2)
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(NB, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    f8_substep<FM, FN, BM>(acc, F[1], F[0], an, bn, xo[0], xo[1], true, da, oa + kof(kt + 2),
                           abuf + (kt & 1) * SA, wave_u);
    b3 = b3n;
  }
  // the trailing re-reads must land before the LDS is reused or released
  wait_dma();
  __syncthreads();
}

// p.A, p.B: the packed code matrices as 16-bit units (p.lda = p.ldb = Kp/2,
// p.K = Kp/2); p.tilesM x p.tilesN tiles cover them exactly; p.M, p.N are
// the output's extent (the epilogue stores only those).
template <int BM, int BN, int EPI>
__global__ void __launch_bounds__(kThreads, 1) gemm_f8_kernel(GemmParams p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int SA = BM * kBK, SB = BN * kBK;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * SA + 3 * SB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
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
  const int b_local = (wn * WN + lc) * kBK;
  int xo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) xo[s] = ((2 * s + h) ^ swz(lc)) << 3;
  f8_mainloop<BM, BN, FM, FN>(p, m0, n0, p.K / kBK, lds, wave, lane, a_base, b_local, xo, acc);
  epilogue<EPI, FM, FN>(p, acc, m0, n0, wm * WM, wn * WN, 0, lane);
}

template <int BM, int BN>
hipError_t launch_f8_tpl(int epi, const GemmParams& p, hipStream_t s) {
  const dim3 grid(p.tilesM * p.tilesN), block(kThreads);
  if (epi == kEpiOsBf16)
    hipLaunchKernelGGL((gemm_f8_kernel<BM, BN, kEpiOsBf16>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((gemm_f8_kernel<BM, BN, kEpiOsF32>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_f8(int tile, int epi, const GemmParams& p, hipStream_t s) {
  if (epi != kEpiOsBf16 && epi != kEpiOsF32) return hipErrorInvalidValue;
  switch (tile) {
    case kF8Tile256x256: return launch_f8_tpl<256, 256>(epi, p, s);
    case kF8Tile256x192: return launch_f8_tpl<256, 192>(epi, p, s);
    case kF8Tile128x128: return launch_f8_tpl<128, 128>(epi, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tgemm
