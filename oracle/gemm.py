"""Oracle GEMM: op(A)·op(B) in fp64 (test infrastructure only).

Follows "Strength reduction: fold transpose into a subsequent GEMM call"
(the program and its trace): the weight is transposed into a new contiguous
array first and only then multiplied; the fast path must reach the same
result without that copy.  Storage is row-major with a leading dimension
(row stride, in elements):

  A 'N': stored [M, K], element (m, k) at A[m*lda + k]
  A 'T': stored [K, M], element (m, k) at A[k*lda + m]
  B 'N': stored [K, N], element (k, n) at B[k*ldb + n]
  B 'T': stored [N, K], element (k, n) at B[n*ldb + k]   (the weight layout)

Operands arrive as flat arrays of bf16 bit patterns and are decoded exactly.
The product is one fp64 matrix multiplication (a library primitive) of the
two explicitly materialised operands; no blocking or reordering beyond that.
"""

import numpy as np

from .bf16 import bf16_bits_to_f64


def _stored_matrix(flat_bits, rows, cols, ld):
    """Decode a row-major [rows, cols] matrix with row stride ``ld``."""
    if ld < cols:
        raise ValueError("leading dimension smaller than row length")
    flat = np.asarray(flat_bits).reshape(-1)
    need = (rows - 1) * ld + cols
    if flat.size < need:
        raise ValueError("operand buffer too small for its shape and ld")
    if flat.size < rows * ld:
        flat = np.concatenate([flat, np.zeros(rows * ld - flat.size, flat.dtype)])
    return bf16_bits_to_f64(flat[: rows * ld].reshape(rows, ld)[:, :cols])


def op_matrix(flat_bits, trans, outer, inner, ld):
    """Materialise op(X) as a fresh contiguous fp64 array.

    For the A operand ``outer``=M and ``inner``=K and the result is [M, K];
    'T' means the stored array is [K, M] and is transposed into a copy.
    For B pass ``outer``=N, ``inner``=K and transpose the returned [N, K]
    via ``gemm``'s handling; see there.
    """
    t = trans.upper()
    if t == "N":
        return np.ascontiguousarray(_stored_matrix(flat_bits, outer, inner, ld))
    if t == "T":
        return np.ascontiguousarray(_stored_matrix(flat_bits, inner, outer, ld).T)
    raise ValueError("trans must be 'N' or 'T'")


def gemm(transA, transB, M, N, K, A_bits, lda, B_bits, ldb, rows=None):
    """C = op(A)·op(B) in fp64, shape [M, N] (or [len(rows), N]).

    ``rows`` optionally selects output rows (sampled parity at full size);
    the selected rows of op(A) are multiplied by the whole op(B).
    """
    opA = op_matrix(A_bits, transA, M, K, lda)          # [M, K]
    tb = transB.upper()
    if tb == "N":
        opB = np.ascontiguousarray(_stored_matrix(B_bits, K, N, ldb))      # [K, N]
    elif tb == "T":
        opB = np.ascontiguousarray(_stored_matrix(B_bits, N, K, ldb).T)    # explicit copy
    else:
        raise ValueError("trans must be 'N' or 'T'")
    if rows is not None:
        opA = opA[np.asarray(rows)]
    return opA @ opB
