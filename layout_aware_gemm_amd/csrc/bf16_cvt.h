// fp32 <-> bf16 on gfx950.  v_cvt_pk_bf16_f32 rounds two fp32 values to
// bf16 with round-to-nearest-even (the default rounding mode of every
// kernel here) and keeps NaN a NaN; bf16 -> fp32 is exact (a shift).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tgemm {

typedef float cvt_f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 cvt_bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 bits of lo in bits 0..15 and of hi in bits 16..31.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const cvt_f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, cvt_bf16x2_t));
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float from_bf16(uint32_t b) { return __uint_as_float(b << 16); }

}  // namespace tgemm
