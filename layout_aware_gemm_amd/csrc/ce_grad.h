// One element of the cross-entropy gradient softmax - onehot from what the
// fused CE GEMM leaves behind ("Allow reductions in matmul epilogues", the
// edit note: the softmax-minus-one-hot matrix kept for the backward pass):
// the stored e = bf16(exp(y - m_b)) of the element, the scale
// s = exp(m_b - lse) of its row and column block, and whether it is the
// label column.  One fused multiply-add, rounded once: e * s - [label].
// Both the rescale pass and the backward GEMMs that apply the rescale while
// loading the gradient use this, so the two routes give the same bits.
#pragma once

#include "bf16_cvt.h"

namespace tgemm {

__device__ __forceinline__ float ce_grad_value(uint32_t e_bits, float s, bool label) {
  return __fmaf_rn(from_bf16(e_bits), s, label ? -1.f : 0.f);
}

// Width (columns) of the blocks of the exported scale table; every CE
// block width (64 or 128) is a multiple of it.
constexpr int kCeScaleCols = 64;

}  // namespace tgemm
