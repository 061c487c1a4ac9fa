// Internal declarations shared by the host dispatcher and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tgemm {

// Epilogue variants of the matrix-core GEMM kernel.  The Q8 stores take
// operands cast to e4m3fn on load (scale, clamp, round) and multiply the
// sum by the output scale before storing.  The OS stores multiply by the
// output scale too, after the fp8 matrix-core kernel (launch_gemm_f8)
// multiplied codes that a separate pass cast (launch_q8_pack).
enum EpiKind : int {
  kEpiStoreBf16 = 0,
  kEpiStoreF32 = 1,
  kEpiCE = 2,
  kEpiQ8Bf16 = 3,
  kEpiQ8F32 = 4,
  kEpiOsBf16 = 5,
  kEpiOsF32 = 6,
  // A is a cross-entropy gradient kept unscaled (see GemmParams::gscale):
  // each loaded element of A becomes bf16(e * s - [label]) before use.
  kEpiGStoreBf16 = 7,
  kEpiGStoreF32 = 8
};

// Tile configurations of the GEMM kernel (k-step 64), 4 waves in a 2x2
// grid: BM x BN = 256x256, 128x128, or 192x256 (NT store epilogues only).
enum TileCfg : int { kTileAuto = 0, kTile256 = 1, kTile128 = 2, kTile192 = 3 };

struct GemmParams {
  const uint16_t* A;  // bf16 bits
  const uint16_t* B;  // bf16 bits
  int64_t lda, ldb, ldc;
  int M, N, K;
  int tilesM, tilesN, groupM;
  int splitk;         // K chunks per tile (1 = no split; store epilogues only)
  int kchunk;         // elements of K per chunk (multiple of 64)
  float* ws;          // split-K partial products: [splitk][M][N] fp32
  int aligned;        // A, B 16-byte aligned and lda, ldb multiples of 8
  void* C;            // store epilogues
  // cross-entropy epilogue
  const int32_t* labels;
  float* part_m;      // [nColBlocks][M] block max
  float* part_s;      // [nColBlocks][M] block sum of exp(y - block max)
  float* ylabel;      // [M] logit at the label column
  uint16_t* grad;     // optional [M][ldc] bf16: exp(y - block max), fixed up later
  // Q8 epilogues: device fp32 {scale_a, scale_b, out_scale}
  const float* qscales;
  // G epilogues: operand A holds e = bf16(exp(y - m_b)) of a fused CE with
  // gtok rows (tokens) and gvoc columns (vocabulary); row t's 64-column
  // chunk c has the scale gscale[c * gtok + t] and the label glabels[t].
  // With A 'N' the GEMM's rows are tokens and its k the vocabulary; with
  // A 'T' the other way round.
  const float* gscale;
  const int32_t* glabels;
  int gtok, gvoc;
};

// Width (in columns) of the per-row partial blocks the CE epilogue writes.
inline int ce_block_cols(int cfg) { return cfg == kTile256 ? 128 : 64; }
inline int tile_rows(int cfg) { return cfg == kTile128 ? 128 : cfg == kTile192 ? 192 : 256; }
inline int tile_cols(int cfg) { return cfg == kTile128 ? 128 : 256; }

// One launcher per operand layout (defined in gemm_<layout>.hip).
hipError_t launch_gemm_nn(int cfg, int epi, const GemmParams& p, hipStream_t s);
hipError_t launch_gemm_nt(int cfg, int epi, const GemmParams& p, hipStream_t s);
hipError_t launch_gemm_tn(int cfg, int epi, const GemmParams& p, hipStream_t s);
hipError_t launch_gemm_tt(int cfg, int epi, const GemmParams& p, hipStream_t s);

// Split-K: C = sum over chunks q = 0, 1, ..., split-1 (in that order) of
// the fp32 partial products ws[q][M][N] (defined in splitk.hip).
hipError_t launch_splitk_sum(const float* ws, int split, int M, int N, void* C, int64_t ldc,
                             bool out_f32, hipStream_t s);

// Matrix-vector and dot products (M = 1 or N = 1, K > 1; defined in
// gemv.hip).  The matrix operand X holds L output rows of K elements:
// kGemvRows when each row is contiguous (row r at X + r*ldx, element k at
// stride sx), kGemvCols when X is stored [K][L] (element (k, r) at
// X + k*ldx + r).  v is the K-vector (stride sv).  gemv_chunks gives the
// number of K chunks, whose fp32 partials [chunks][L] `partial` must hold;
// the result r is stored at C + r*sc.
enum GemvShape : int { kGemvRows = 0, kGemvCols = 1 };
int64_t gemv_chunks(int shape, int L, int64_t K);
hipError_t launch_gemv(int shape, const uint16_t* X, int64_t ldx, int64_t sx, const uint16_t* v,
                       int64_t sv, int L, int64_t K, int nkc, float* partial, void* C,
                       int64_t sc, bool out_f32, hipStream_t s);

// Cross-entropy combine (per row: fold block partials in ascending block
// order, loss = lse - y[label]) and gradient fix-up (defined in ce.hip).
hipError_t launch_ce_combine(const float* part_m, const float* part_s, const float* ylabel,
                             const int32_t* labels, int M, int N, int nblk, float* loss,
                             float* lse, hipStream_t s);
// The deferred gradient's scale table, fp32 [ceil(N/64)][M] (ce.hip).
hipError_t launch_ce_scale(const float* part_m, const float* lse, int M, int N, int blk_cols,
                           float* scale, hipStream_t s);
hipError_t launch_ce_grad_fixup(uint16_t* grad, int64_t ldc, const float* part_m,
                                const float* lse, const int32_t* labels, int M, int N,
                                int blk_cols, hipStream_t s);

// K = 1 pointwise paths (defined in k1.hip).  Strides are element strides
// of the length-M vector a and the length-N vector b.
hipError_t launch_k1_rope(const int64_t* pos, int64_t spos, const float* invf, int64_t sinv,
                          int M, int N, uint16_t* cos_out, uint16_t* sin_out, int64_t ldc,
                          hipStream_t s);
hipError_t launch_k1_outer_f32(const float* a, int64_t sa, const float* b, int64_t sb, int M,
                               int N, float* C, int64_t ldc, hipStream_t s);
hipError_t launch_k1_outer_bf16(const uint16_t* a, int64_t sa, const uint16_t* b, int64_t sb,
                                int M, int N, void* C, int64_t ldc, bool out_f32, hipStream_t s);
// The RoPE region in one launch: the cos / sin tables (D = 2F columns, F
// = D/2 inverse frequencies, contiguous) of P positions, and the query q
// [P, ldq] bf16 (H heads of D) widened and permuted into q_out fp32
// [H][P][D] (defined in k1.hip).
hipError_t launch_rope_region(const uint16_t* q, int64_t ldq, int64_t P, int64_t H, int64_t D,
                              const int64_t* pos, int64_t spos, const float* invf,
                              uint16_t* cos_out, uint16_t* sin_out, int64_t ldc, float* q_out,
                              hipStream_t s);
// Cross-entropy of the K = 1 logits y[m, n] = a[m] * b[n] (bf16 operands):
// loss[m] = logsumexp_n y - y[m, labels[m]]; grad (optional, row stride ldg)
// = bf16(softmax - onehot).  One workgroup per row.
hipError_t launch_k1_ce(const uint16_t* a, int64_t sa, const uint16_t* b, int64_t sb, int M,
                        int N, const int32_t* labels, float* loss, uint16_t* grad, int64_t ldg,
                        hipStream_t s);

// e4m3fn cast (scale[0], clamp, round) of an fp8 GEMM operand into the
// K-contiguous code matrix out [Rp][Kp] (one byte per code, zero past R
// rows and K columns) that launch_gemm_f8 reads.  k_contiguous: X is [R][K]
// with row stride ld (K % 8 == 0); otherwise X is [K][R] with row stride ld
// (R % 8 == 0).  X 16-byte aligned, ld % 8 == 0, Rp % 64 == 0, Kp % 128 == 0.
struct PackOperand {
  const uint16_t* X;
  int64_t ld;
  bool k_contiguous;
  int R, K;
  const float* scale;
  uint8_t* out;
  int Rp, Kp;
};
// Both operands of one product in one launch (defined in fp8_cast.hip).
hipError_t launch_q8_pack(const PackOperand& a, const PackOperand& b, hipStream_t s);

// fp8 matrix-core GEMM over two packed code matrices (defined in
// gemm_f8.hip): p.A [tilesM*BM][2*p.K] and p.B [tilesN*BN][2*p.K] bytes
// passed as 16-bit units (p.lda = p.ldb = p.K, p.K % 64 == 0), an OS
// epilogue, C [p.M][p.N].  tile: one of the F8Tile shapes (BM x BN).
enum F8Tile : int { kF8Tile256x256 = 0, kF8Tile256x192 = 1, kF8Tile128x128 = 2 };
inline int f8_tile_rows(int t) { return t == kF8Tile128x128 ? 128 : 256; }
inline int f8_tile_cols(int t) { return t == kF8Tile256x256 ? 256 : t == kF8Tile256x192 ? 192 : 128; }
hipError_t launch_gemm_f8(int tile, int epi, const GemmParams& p, hipStream_t s);

}  // namespace tgemm
