/*
 * tgemm -- layout-aware bf16 GEMM for MI355X (gfx950) with fused epilogues.
 *
 * One C-ABI library.  Plain pointers and sizes only; every data pointer is a
 * DEVICE pointer owned by the caller, and every call is asynchronous on the
 * caller's HIP stream.
 *
 * What is computed
 * ----------------
 *   Y = op(A) . op(B),  op(X) = X for 'N' and X^T for 'T'.
 *
 *   The transpose is a flag, never a copy: a weight stored [N,K] row-major is
 *   read in place as op(B) with transB = 'T' ("Strength reduction: fold
 *   transpose into a subsequent GEMM call", the trace and its discussion of
 *   NT GEMMs; the pitch asks for GEMMs that take transpose arguments).
 *
 * Storage convention (row-major, leading dimension = row stride in elements)
 *   A 'N': [M,K], element (m,k) at A[m*lda + k]     lda >= K
 *   A 'T': [K,M], element (m,k) at A[k*lda + m]     lda >= M
 *   B 'N': [K,N], element (k,n) at B[k*ldb + n]     ldb >= N
 *   B 'T': [N,K], element (k,n) at B[n*ldb + k]     ldb >= K
 *   C    : [M,N], element (m,n) at C[m*ldc + n]     ldc >= N (>= 2N for ROPE)
 *
 * Epilogues (argument `epilogue`)
 *   TGEMM_EPI_STORE_BF16   A, B bf16 -> C bf16, fp32 accumulation, output
 *                          rounded to nearest even.
 *   TGEMM_EPI_STORE_F32    A, B bf16 -> C fp32 (the raw accumulator).
 *   TGEMM_EPI_CE           A, B bf16; the logits y = op(A).op(B) (fp32) are
 *                          reduced per row and never written out:
 *                            loss[m] = logsumexp_n y[m,n] - y[m, labels[m]]
 *                          written to out_loss (fp32[M]).  If out_grad is not
 *                          NULL it receives softmax(y) - onehot(labels) as
 *                          bf16 [M,N] with row stride ldc.  C is ignored.
 *                          ("Allow reductions in matmul epilogues": the
 *                          attempted fusion defines the max / exp / sum / log
 *                          steps, the loss and the softmax-minus-one-hot
 *                          output; its answer on tile-wise row reductions
 *                          describes the cross-tile combine.)
 *                          Labels outside [0,N) are not checked on the host:
 *                          that row's loss is NaN and its gradient row is the
 *                          plain softmax.  No mean over rows, no scaling.
 *   TGEMM_EPI_OUTER_F32    K must be 1.  A, B fp32; C fp32 [M,N] = the exact
 *                          fp32 products a[m]*b[n].
 *   TGEMM_EPI_ROPE_COSSIN  K must be 1.  A int64 positions (cast to fp32 in
 *                          the kernel; exact for |p| < 2^24), B fp32 inverse
 *                          frequencies.  t = fp32(a[m]) * b[n];
 *                          C        = cos(t) as bf16 at columns n and n+N,
 *                          out_grad = sin(t) as bf16 at columns n and n+N,
 *                          both [M, 2N] with row stride ldc.
 *                          ("Schedule a small matmul op as a reduction (or
 *                          pointwise) op": the %kernel_math listing's K=1
 *                          matmul, permute, duplicating cat and cos/cast, and
 *                          the proposed broadcast-multiply decomposition.)
 *
 *   Every call with K == 1 runs pointwise, without matrix cores, as that
 *   page proposes for K=1 matmuls: the STORE epilogues as an outer product,
 *   CE as a per-row reduction of the logits a[m]*b[n] (bf16 operands, the
 *   products exact in fp32).
 *
 * Errors
 *   Arguments are validated before anything is enqueued; on any error
 *   nothing is written.  No exceptions cross the ABI.  The call returns
 *   after enqueueing and never synchronises; faults inside a kernel surface
 *   at the caller's next synchronisation.  Outputs must not alias inputs.
 *
 * Workspace
 *   TGEMM_EPI_CE needs a small scratch buffer (per row and per 128-column
 *   block: the block max and block sum of exponentials, plus per row the
 *   label logit and the logsumexp).  A store-epilogue GEMM whose tiles
 *   alone do not fill the GPU (few output tiles, long K; both operands
 *   K-contiguous) splits K into chunks and needs one fp32 M x N partial
 *   product per chunk; a second kernel adds them in chunk order.
 *   The library keeps one workspace buffer per (device, stream): calls on
 *   a stream run in order and reuse it; it grows with hipFreeAsync /
 *   hipMallocAsync on that stream, so calls on different streams never
 *   share memory.  While `stream` is being captured into a graph the call
 *   allocates and frees its own buffer in stream order instead.
 *
 * Threads
 *   tgemm_run may be called from several host threads, on the same stream
 *   or on different ones.  A call holds its stream's workspace entry from
 *   the lookup until its last kernel is enqueued, so concurrent calls on
 *   one stream are enqueued one after the other and never see a buffer
 *   freed under them.  The tuning knobs (tgemm_set_*) are process-wide and
 *   must not change while calls are in flight.
 *
 * Retention
 *   A stream's cached buffer is held until the process ends or until
 *   tgemm_release_workspace(stream) frees it; a program that creates many
 *   short-lived streams should release each one's buffer before destroying
 *   the stream.  A stream must not be destroyed while a tgemm call on it is
 *   still executing.
 */
#ifndef TGEMM_H
#define TGEMM_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define TGEMM_API __attribute__((visibility("default")))
#else
#define TGEMM_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TGEMM_OK = 0,
  TGEMM_ERR_INVALID_ARG = -1, /* a flag, size, leading dimension or pointer is invalid */
  TGEMM_ERR_UNSUPPORTED = -2, /* valid request this library does not implement      */
  TGEMM_ERR_HIP = -3,         /* the HIP runtime reported an error while enqueueing   */
  TGEMM_ERR_NO_MEMORY = -4,   /* a CE or split-K workspace could not be allocated     */
  TGEMM_ERR_WORKSPACE_LIMIT = -5 /* tgemm_run_noalloc: the call needs more scratch than
                                    its fixed buffer holds (tgemm_noalloc_scratch_bytes) */
} tgemm_status;

typedef enum {
  TGEMM_EPI_STORE_BF16 = 0,
  TGEMM_EPI_STORE_F32 = 1,
  TGEMM_EPI_CE = 2,
  TGEMM_EPI_OUTER_F32 = 3,
  TGEMM_EPI_ROPE_COSSIN = 4
} tgemm_epilogue;

/*
 * Run one GEMM with the chosen epilogue on `stream` (a hipStream_t; NULL is
 * the null stream).
 *
 *   transA, transB  'N'/'n' or 'T'/'t' (see the storage convention above).
 *   M, N, K         >= 1 and < 2^31.
 *   A, lda          operand A (bf16; fp32 for OUTER_F32; int64 for ROPE).
 *   B, ldb          operand B (bf16; fp32 for OUTER_F32 and ROPE).
 *   C, ldc          output (bf16 or fp32; cos table for ROPE; unused by CE).
 *                   For CE, ldc is the row stride of out_grad.
 *   labels          CE only: int32[M].
 *   out_loss        CE only: fp32[M].
 *   out_grad        CE: optional bf16 [M,N] (row stride ldc);
 *                   ROPE: required sin table bf16 [M,2N] (row stride ldc).
 *
 * Returns TGEMM_OK or a negative tgemm_status.
 */
TGEMM_API int tgemm_run(char transA, char transB, int64_t M, int64_t N, int64_t K,
              const void* A, int64_t lda, const void* B, int64_t ldb,
              void* C, int64_t ldc, int epilogue,
              const int32_t* labels, float* out_loss, void* out_grad,
              void* stream);

/*
 * tgemm_run without allocation, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, results and errors as tgemm_run (the
 * same kernels), but every scratch buffer the call needs -- the split-K
 * partial products, the cross-entropy block partials, the matrix-vector
 * partials -- lives in one fixed device array of the library,
 * tgemm_noalloc_scratch_bytes() = 64 MiB per device, held from the first
 * use on a device until the process ends.  The call makes no hipMalloc,
 * hipFree or other allocating call; the caller still owns every input and
 * output.  A call whose scratch need exceeds the array returns
 * TGEMM_ERR_WORKSPACE_LIMIT before anything is enqueued (the 768x5120x13824
 * NT product needs 45 MiB: 3 K chunks; split-K needs 4*chunks*M*N bytes, cross-entropy
 * about 8*M*(N/128 + 1) bytes).
 *
 * Every call on a device shares that device's array, and the array keeps
 * the last call's contents (no kernel relies on them: each writes every
 * scratch value it reads).  Calls that may overlap on one device -- on two
 * streams, or from two threads -- race on the array and give wrong
 * results; serialise them (one stream, in order) or use tgemm_run.
 */
TGEMM_API int tgemm_run_noalloc(char transA, char transB, int64_t M, int64_t N, int64_t K,
                                const void* A, int64_t lda, const void* B, int64_t ldb,
                                void* C, int64_t ldc, int epilogue,
                                const int32_t* labels, float* out_loss, void* out_grad,
                                void* stream);

/* Size in bytes of tgemm_run_noalloc's fixed scratch array. */
TGEMM_API int64_t tgemm_noalloc_scratch_bytes(void);

/*
 * Host-only argument check with the same rules as tgemm_run, without
 * touching the GPU.  Returns TGEMM_OK or the status tgemm_run would return.
 */
TGEMM_API int tgemm_validate(char transA, char transB, int64_t M, int64_t N, int64_t K,
                   const void* A, int64_t lda, const void* B, int64_t ldb,
                   const void* C, int64_t ldc, int epilogue,
                   const int32_t* labels, const float* out_loss,
                   const void* out_grad);

/*
 * GEMM on fp8 (e4m3fn) operands made on the fly from bf16 inputs.
 *
 * ("Improve the Inductor generated kernel for the pattern of output1 =
 * pointwise(input); output2 = transpose(output1)", the example: before a
 * float8 linear each input element is scaled, clamped to the largest
 * finite e4m3fn value and cast to e4m3fn, and the page's pattern also
 * writes a transposed copy of the fp8 tensor.  Here no transposed copy is
 * ever stored: the operands are read in their stored layouts.)
 *
 *   transA, transB, M, N, K, A, lda, B, ldb, C, ldc: as for tgemm_run with
 *                   a STORE epilogue; A and B are bf16 in any layout.
 *   epilogue        TGEMM_EPI_STORE_BF16 or TGEMM_EPI_STORE_F32 only.
 *   scales          device pointer to three fp32 values
 *                   {scale_a, scale_b, out_scale}, read by the kernel.
 *
 * Each element x of op(A) becomes q = e4m3fn(clamp(fp32(x) * scale_a,
 * -448, 448)): one fp32 multiply, the clamp (NaN stays NaN), then rounding
 * to nearest e4m3fn value with ties to even; likewise op(B) with scale_b.
 * C = out_scale * sum_k qA[m,k] * qB[k,n], products exact, fp32
 * accumulation, one fp32 multiply by out_scale, then the store epilogue
 * (bf16 with round-to-nearest-even, or fp32).  Pass out_scale =
 * 1 / (scale_a * scale_b) to undo both casts.
 *
 * Large products (at least two 256-row and two 256-column tiles, every
 * stored row 16-byte aligned with a multiple of 8 elements) cast each
 * operand once into a K-contiguous matrix of e4m3fn codes (one byte each,
 * zero-padded to whole tiles) in the library's per-stream workspace, and
 * multiply the codes on the fp8 matrix cores (v_mfma_f32_32x32x64_f8f6f4).
 * Other products cast each element as the GEMM loads it and multiply on
 * the bf16 matrix cores, which hold every e4m3fn value exactly.  Both
 * routes multiply the same e4m3fn values with fp32 accumulation; their
 * sums may differ in the last bits (the matrix cores group the k
 * differently), and both are exact where every partial sum is exactly
 * representable (e.g. integer-valued operands).  tgemm_set_fp8_cast_once(0)
 * forces the cast on load.  If the workspace for the codes cannot be
 * allocated, the product casts on load.
 *
 * Validation, errors, asynchrony and streams as for tgemm_run.  Returns
 * TGEMM_OK or a negative tgemm_status; an unsupported epilogue or a NULL
 * `scales` is TGEMM_ERR_INVALID_ARG.
 */
TGEMM_API int tgemm_run_fp8(char transA, char transB, int64_t M, int64_t N, int64_t K,
                  const void* A, int64_t lda, const void* B, int64_t ldb,
                  void* C, int64_t ldc, int epilogue, const float* scales,
                  void* stream);

/* Host-only argument check of tgemm_run_fp8 (no GPU access). */
TGEMM_API int tgemm_validate_fp8(char transA, char transB, int64_t M, int64_t N, int64_t K,
                  const void* A, int64_t lda, const void* B, int64_t ldb,
                  const void* C, int64_t ldc, int epilogue, const float* scales);

/*
 * Cross-entropy with the gradient left for the backward GEMMs to finish
 * ("Allow reductions in matmul epilogues", the edit note: the
 * softmax-minus-one-hot matrix is kept for the backward pass).
 *
 * As tgemm_run with TGEMM_EPI_CE and a gradient buffer (same arguments,
 * same loss, bit for bit), except that the pass that rescales the gradient
 * is not run.  Instead:
 *   out_e      bf16 [M, N] (row stride lde >= N) receives
 *              e = bf16(exp(y - m_b)), y the fp32 logit and m_b the maximum
 *              of y over the block of columns the GEMM's tile reduced (64 or
 *              128 columns);
 *   out_scale  fp32 [ceil(N/64) * M] receives, for every 64-column chunk c
 *              of every row m, s[c*M + m] = exp(m_b - lse[m]) of the block
 *              holding the chunk.
 * The gradient is then softmax - onehot = bf16(e * s - [n == labels[m]])
 * (one fused multiply-add, rounded once), which tgemm_run_ce_grad computes
 * as it loads e, and which equals bit for bit what the rescale pass of
 * tgemm_run writes.  K must be >= 2 (a K = 1 product takes the pointwise
 * path, which has no deferred form): TGEMM_ERR_UNSUPPORTED otherwise.
 * Validation, errors, asynchrony, streams and workspace as for tgemm_run.
 */
TGEMM_API int tgemm_run_ce_deferred(char transA, char transB, int64_t M, int64_t N, int64_t K,
                                    const void* A, int64_t lda, const void* B, int64_t ldb,
                                    const int32_t* labels, float* out_loss, void* out_e,
                                    int64_t lde, float* out_scale, void* stream);

/*
 * A GEMM whose operand A is a cross-entropy gradient left by
 * tgemm_run_ce_deferred, finished as it is loaded:
 *   C = op(G) . op(B),  G[t][v] = bf16(e[t*lde + v] * scale[(v/64)*T + t]
 *                                      - [v == labels[t]])
 * with G a [T, V] matrix (T token rows, V vocabulary columns) stored as e:
 * transA 'N' reads it as op(A) = G (T = M, V = K; the gradient of the
 * hidden states, dH = G . W), 'T' as op(A) = G^T (T = K, V = M; the
 * gradient of the weight, dW = G^T . H).  B, transB, ldb, C, ldc as for
 * tgemm_run; epilogue TGEMM_EPI_STORE_BF16 or TGEMM_EPI_STORE_F32.  Every
 * shape runs on the matrix-core kernel (no pointwise, matrix-vector or
 * split-K route).  The result equals, bit for bit, tgemm_run on the
 * gradient the rescale pass writes.  Labels outside [0, V) subtract
 * nothing.  Validation, errors, asynchrony and streams as for tgemm_run; a
 * NULL scale or labels, or another epilogue, is TGEMM_ERR_INVALID_ARG.
 */
TGEMM_API int tgemm_run_ce_grad(char transA, char transB, int64_t M, int64_t N, int64_t K,
                                const void* E, int64_t lde, const float* scale,
                                const int32_t* labels, const void* B, int64_t ldb, void* C,
                                int64_t ldc, int epilogue, void* stream);

/*
 * The RoPE region of "Schedule a small matmul op as a reduction (or
 * pointwise) op" as far as that page's %kernel_math listing goes, in one
 * launch (the page's closing remark: the section fused into a single
 * kernel, the K = 1 matmul included):
 *   - the cos / sin tables of the positions, exactly as tgemm_run with
 *     TGEMM_EPI_ROPE_COSSIN and K = 1: t = fp32(pos[p]) * inv_freq[i]
 *     (i < F = D/2), cos_out / sin_out[p, i] and [p, i + F] = bf16(cos t) /
 *     bf16(sin t) (the listing's T19 .. T26 and the second table output);
 *   - the query of the listing's first three steps: q [P, ldq] bf16, row p
 *     holding H heads of D values (head h at columns h*D .. h*D + D-1),
 *     viewed as [P, H, D] (T5), permuted to [H, P, D] (T6) and widened to
 *     fp32 (T34), written to q_out[(h*P + p)*D + d] (fp32, contiguous
 *     [H][P][D]).
 * The rotation that turns these into the region's rotated outputs is not
 * on the page and is not applied.
 *
 *   q, ldq        bf16 query rows, ldq >= H*D (elements).
 *   P, H, D       positions, heads, head width; P, H >= 1, D >= 2 even.
 *   pos, spos     int64 positions, element stride spos >= 1.
 *   inv_freq      fp32 [D/2], contiguous.
 *   cos_out, sin_out  bf16 [P, ldc], ldc >= D.
 *   q_out         fp32 [H*P*D].
 * All pointers are device pointers owned by the caller; outputs must not
 * alias inputs.  Validation, errors, asynchrony and streams as for
 * tgemm_run; no workspace.  Returns TGEMM_OK or a negative tgemm_status.
 */
TGEMM_API int tgemm_rope_region(const void* q, int64_t ldq, int64_t P, int64_t H, int64_t D,
                                const int64_t* pos, int64_t spos, const float* inv_freq,
                                void* cos_out, void* sin_out, int64_t ldc, float* q_out,
                                void* stream);

/* Host-only argument check of tgemm_rope_region (no GPU access). */
TGEMM_API int tgemm_validate_rope_region(const void* q, int64_t ldq, int64_t P, int64_t H,
                                         int64_t D, const int64_t* pos, int64_t spos,
                                         const float* inv_freq, const void* cos_out,
                                         const void* sin_out, int64_t ldc, const float* q_out);

/* Human-readable name of a status code (static string, never NULL). */
TGEMM_API const char* tgemm_status_string(int status);

/*
 * Tuning / testing knob: force the GEMM tile configuration for subsequent
 * calls from this process.  0 = automatic (default); 1 = 256x256 tiles;
 * 2 = 128x128 tiles; 3 = 192x256 tiles for NT products with a store
 * epilogue (256x256 for any other call).  Returns the previous value, or
 * TGEMM_ERR_INVALID_ARG for an unknown value.
 * Not thread-safe with concurrent tgemm_run calls.
 */
TGEMM_API int tgemm_set_tile_config(int config);

/*
 * Tuning / testing knob: force the number of K chunks a GEMM with a store
 * epilogue is split into (each chunk is a separate workgroup writing an
 * fp32 partial product; a second kernel adds the partials in ascending
 * chunk order, so results do not depend on timing).  Ignored for the CE
 * epilogue.  0 = automatic (default), 1 = never
 * split.  Returns the previous value, or TGEMM_ERR_INVALID_ARG outside
 * 0..64.  Not thread-safe with concurrent tgemm_run calls.
 */
TGEMM_API int tgemm_set_split_k(int split);

/*
 * Tuning / testing knob for tgemm_run_fp8: 1 (default) lets large products
 * (at least two 256-row and two 256-column tiles, 16-byte rows) cast each
 * operand once, in a pass of its own, into K-contiguous e4m3fn codes in the
 * library's per-stream workspace and multiply them on the fp8 matrix
 * cores; 0 always casts on load (bf16 matrix cores).  Both routes multiply
 * the same e4m3fn values; their fp32 sums may differ in the last bits.
 * Returns the previous value,
 * or TGEMM_ERR_INVALID_ARG for anything but 0 or 1.  Not thread-safe with
 * concurrent tgemm_run_fp8 calls.
 */
TGEMM_API int tgemm_set_fp8_cast_once(int enable);

/*
 * Measurement aid, beside the GEMM path: the shader clock the device runs
 * at.  Enqueues on `stream` one wave that polls the device's constant-rate
 * counter until it has advanced by `ticks` (1 <= ticks <= 10^7; at the
 * usual 100 MHz rate, 2000 ticks = 20 us), then writes three uint64 values
 * to out_ticks (device memory, 8-byte aligned, owned by the caller): the
 * shader-clock cycles that elapsed, the constant-rate ticks that elapsed,
 * and the constant rate in Hz.  The shader clock over the wait is
 * out[0] * out[2] / out[1].  Enqueued right after a timed region it reads
 * the clock that region ended at.  Asynchronous like tgemm_run.  Returns
 * TGEMM_OK, TGEMM_ERR_INVALID_ARG (ticks out of range, NULL or misaligned
 * out_ticks; checked before any device call) or TGEMM_ERR_HIP.
 */
TGEMM_API int tgemm_clock_probe(int64_t ticks, uint64_t* out_ticks, void* stream);

/*
 * Matrix-core ceiling (a measurement aid, not part of the GEMM path):
 * enqueue `blocks` workgroups of 4 waves (one workgroup per compute unit,
 * one wave per SIMD) that each issue only MFMAs on operands held in
 * registers: `iters` iterations of 16 MFMAs into 16 independent 32x32
 * accumulator blocks.  kind 0: v_mfma_f32_32x32x16_bf16 on finite bf16
 * values, 524288 flop per wave and iteration; kind 1: the 32x32x64 MFMA on
 * fp8 e4m3fn codes (never NaN), 2097152 flop.  The work is blocks * 4 *
 * iters times that; timing it on `stream` gives the matrix-core rate
 * without loads, LDS or barriers at the clock the chip holds under it.
 * `out` (device, float[blocks * 4], 4-byte aligned, caller-owned) receives
 * element 0 of block 0 of each wave, so the work is kept (iters = 2 gives
 * twice the values of iters = 1 up to the fp32 roundings of the
 * accumulation).  Returns TGEMM_OK, TGEMM_ERR_INVALID_ARG (kind not 0 or
 * 1, iters outside [1, 1e8], blocks outside [1, 65536], NULL or misaligned
 * out; checked before any device call) or TGEMM_ERR_HIP.
 */
TGEMM_API int tgemm_mfma_ceiling(int kind, int64_t iters, int blocks, float* out, void* stream);

/*
 * Free the cached workspace buffer of (current device, `stream`) in stream
 * order (hipFreeAsync on `stream`); the next tgemm_run on that stream
 * allocates a new one.  Work already enqueued keeps a valid buffer.  A
 * stream that has none is a no-op.  Must not race with tgemm_run calls on
 * the same stream from other threads (it waits for a call holding the entry
 * to finish enqueueing).  Returns TGEMM_OK or TGEMM_ERR_HIP.
 */
TGEMM_API int tgemm_release_workspace(void* stream);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
TGEMM_API int tgemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_H */
