// Host-side argument validation for tgemm_run.  Pure C++ (no HIP), so it
// can be built and tested on a machine without a GPU.
#include "tgemm.h"

#include <stdint.h>

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

inline bool flag_ok(char t) { return t == 'N' || t == 'n' || t == 'T' || t == 't'; }
inline bool is_n(char t) { return t == 'N' || t == 'n'; }

}  // namespace

extern "C" int tgemm_validate(char transA, char transB, int64_t M, int64_t N, int64_t K,
                              const void* A, int64_t lda, const void* B, int64_t ldb,
                              const void* C, int64_t ldc, int epilogue,
                              const int32_t* labels, const float* out_loss,
                              const void* out_grad) {
  if (!flag_ok(transA) || !flag_ok(transB)) return TGEMM_ERR_INVALID_ARG;
  if (epilogue < TGEMM_EPI_STORE_BF16 || epilogue > TGEMM_EPI_ROPE_COSSIN)
    return TGEMM_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1) return TGEMM_ERR_INVALID_ARG;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return TGEMM_ERR_UNSUPPORTED;

  // Leading dimensions: the row stride of each stored (row-major) array.
  const int64_t min_lda = is_n(transA) ? K : M;
  const int64_t min_ldb = is_n(transB) ? N : K;
  if (lda < min_lda || ldb < min_ldb) return TGEMM_ERR_INVALID_ARG;
  if (A == nullptr || B == nullptr) return TGEMM_ERR_INVALID_ARG;

  switch (epilogue) {
    case TGEMM_EPI_STORE_BF16:
    case TGEMM_EPI_STORE_F32:
      if (C == nullptr || ldc < N) return TGEMM_ERR_INVALID_ARG;
      break;
    case TGEMM_EPI_CE:
      if (labels == nullptr || out_loss == nullptr) return TGEMM_ERR_INVALID_ARG;
      if (out_grad != nullptr && ldc < N) return TGEMM_ERR_INVALID_ARG;
      break;
    case TGEMM_EPI_OUTER_F32:
      if (K != 1) return TGEMM_ERR_UNSUPPORTED;
      if (C == nullptr || ldc < N) return TGEMM_ERR_INVALID_ARG;
      break;
    case TGEMM_EPI_ROPE_COSSIN:
      if (K != 1) return TGEMM_ERR_UNSUPPORTED;
      if (C == nullptr || out_grad == nullptr) return TGEMM_ERR_INVALID_ARG;
      if (N > kMaxDim / 2 || ldc < 2 * N) return TGEMM_ERR_INVALID_ARG;
      break;
    default:
      return TGEMM_ERR_INVALID_ARG;
  }
  // Row strides times row counts must stay addressable with 64-bit offsets.
  const int64_t rowsA = is_n(transA) ? M : K, rowsB = is_n(transB) ? K : N;
  if (lda > INT64_MAX / rowsA || ldb > INT64_MAX / rowsB || ldc > INT64_MAX / M)
    return TGEMM_ERR_UNSUPPORTED;
  return TGEMM_OK;
}

extern "C" int tgemm_validate_fp8(char transA, char transB, int64_t M, int64_t N, int64_t K,
                                  const void* A, int64_t lda, const void* B, int64_t ldb,
                                  const void* C, int64_t ldc, int epilogue,
                                  const float* scales) {
  if (epilogue != TGEMM_EPI_STORE_BF16 && epilogue != TGEMM_EPI_STORE_F32)
    return TGEMM_ERR_INVALID_ARG;
  if (scales == nullptr) return TGEMM_ERR_INVALID_ARG;
  return tgemm_validate(transA, transB, M, N, K, A, lda, B, ldb, C, ldc, epilogue, nullptr,
                        nullptr, nullptr);
}

extern "C" int tgemm_validate_rope_region(const void* q, int64_t ldq, int64_t P, int64_t H,
                                          int64_t D, const int64_t* pos, int64_t spos,
                                          const float* inv_freq, const void* cos_out,
                                          const void* sin_out, int64_t ldc, const float* q_out) {
  if (P < 1 || H < 1 || D < 2 || (D & 1) != 0) return TGEMM_ERR_INVALID_ARG;
  if (P > kMaxDim || H > kMaxDim || D > kMaxDim) return TGEMM_ERR_UNSUPPORTED;
  if (q == nullptr || pos == nullptr || inv_freq == nullptr || cos_out == nullptr ||
      sin_out == nullptr || q_out == nullptr)
    return TGEMM_ERR_INVALID_ARG;
  if (spos < 1 || ldc < D) return TGEMM_ERR_INVALID_ARG;
  if (H > INT64_MAX / D || ldq < H * D) return TGEMM_ERR_INVALID_ARG;
  if (ldq > INT64_MAX / P || ldc > INT64_MAX / P || spos > INT64_MAX / P ||
      H * D > INT64_MAX / P / 4)
    return TGEMM_ERR_UNSUPPORTED;
  return TGEMM_OK;
}

extern "C" const char* tgemm_status_string(int status) {
  switch (status) {
    case TGEMM_OK: return "TGEMM_OK";
    case TGEMM_ERR_INVALID_ARG: return "TGEMM_ERR_INVALID_ARG";
    case TGEMM_ERR_UNSUPPORTED: return "TGEMM_ERR_UNSUPPORTED";
    case TGEMM_ERR_HIP: return "TGEMM_ERR_HIP";
    case TGEMM_ERR_NO_MEMORY: return "TGEMM_ERR_NO_MEMORY";
    case TGEMM_ERR_WORKSPACE_LIMIT: return "TGEMM_ERR_WORKSPACE_LIMIT";
    default: return "TGEMM_ERR_UNKNOWN";
  }
}

extern "C" int tgemm_version(void) { return 200; }
