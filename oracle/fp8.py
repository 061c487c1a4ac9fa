"""fp8 (e4m3fn) operands made on the fly from bf16 inputs, and the GEMM on them.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Improve the Inductor generated kernel for the pattern of output1 =
pointwise(input); output2 = transpose(output1)", the example.  Before a
float8 linear, each input element is multiplied by a scale in fp32, clamped
to plus or minus the largest finite e4m3fn magnitude, and cast to e4m3fn;
the page's pattern then also writes a transposed copy of the fp8 tensor.
The layout-aware GEMM instead reads the bf16 input in its stored layout and
applies the same scale, clamp and cast as it loads each element, so neither
the fp8 tensor nor its transposed copy exists.

The page fixes the cast, not its consumer.  Reading: the GEMM multiplies
the rounded operands exactly (every product of two e4m3fn values is exact
in fp32) with fp32 accumulation, and multiplies the sum by an output scale
(the caller passes 1 / (scale_a * scale_b) to undo both casts).

e4m3fn, from the format's definition: 1 sign bit, 4 exponent bits with bias
7 and 3 fraction bits.  Exponent fields 1..15 give (1 + f/8) * 2^(e-7), the
field 0 gives the subnormals f/8 * 2^-6, and the single all-ones pattern
(exponent 15, fraction 7) is NaN: there are no infinities.  So the finite
values are spaced 2^(E-3) between 2^E and 2^(E+1) for E >= -6, spaced 2^-9
below 2^-6, and end at 448 = 1.75 * 2^8.  Rounding is to nearest, ties to
the even fraction (the cast's default).
"""

import numpy as np

from .gemm import op_matrix

E4M3_MAX = 448.0


def e4m3_round(y):
    """Round fp32/fp64 values of magnitude <= 448 (or NaN) to e4m3fn values,
    nearest with ties to even; returns fp64.  Larger magnitudes are the
    caller's to clamp first (the format has nothing above 448)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, ex = np.frexp(a)                    # a = m * 2^ex with m in [0.5, 1)
    e = np.maximum(ex - 1, -6)             # exponent of the leading bit; subnormals share -6
    q = np.ldexp(1.0, e - 3)               # spacing of values with 3 fraction bits
    r = np.round(a / q) * q                # a / q is exact (q is a power of two); half to even
    out = np.copysign(r, y)
    return np.where(np.isnan(y), np.nan, out)


def quantize(x, scale):
    """The page's cast of one operand: fp32(x) * fp32(scale) rounded once in
    fp32, clamped to [-448, 448] (NaN stays NaN), then rounded to e4m3fn.
    Returns the e4m3fn values as fp64."""
    y = np.asarray(x, dtype=np.float32) * np.float32(scale)     # fp32 multiply, one rounding
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))  # NaN propagates through clip
    return e4m3_round(y)


def gemm_fp8(transA, transB, M, N, K, A_bits, lda, B_bits, ldb, scale_a, scale_b,
             out_scale=1.0, rows=None):
    """out_scale * (quantize(op(A), scale_a) @ quantize(op(B), scale_b)) in
    fp64, shape [M, N] (or [len(rows), N]).  A and B are bf16 bit patterns in
    their stored layouts; op() as in ``gemm``.  The sum of K products of
    e4m3fn values is exact in fp64 for any K used here (each product has at
    most 8 significant bits and lies in [2^-18, 448^2])."""
    qa = quantize(op_matrix(A_bits, transA, M, K, lda), scale_a)
    tb = transB.upper()
    if tb == "N":
        opB = op_matrix(B_bits, "T", N, K, ldb).T    # stored [K, N]: rows of the transpose
    elif tb == "T":
        opB = op_matrix(B_bits, "N", N, K, ldb).T    # stored [N, K]
    else:
        raise ValueError("trans must be 'N' or 'T'")
    qb = quantize(np.ascontiguousarray(opB), scale_b)
    if rows is not None:
        qa = qa[np.asarray(rows)]
    return (qa @ qb) * np.float64(out_scale)
