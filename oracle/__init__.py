"""CPU oracle for the layout-aware bf16 GEMM and its epilogues.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library or its Python binding and imports neither; both sides receive
the same seeded inputs from the ``workloads`` package, which holds no
arithmetic of the method.

Everything is computed from the plain definitions in fp64 with NumPy:

* ``gemm``        -- op(A)·op(B) by explicit transpose-then-multiply
                     ("Strength reduction: fold transpose into a subsequent
                     GEMM call", the program and its trace).
* ``cross_entropy`` / ``tile_partials`` / ``merge_partials``
                  -- the row-wise cross-entropy of "Allow reductions in
                     matmul epilogues" (the attempted fusion: max, shifted
                     exp, sum, log, loss, softmax minus one-hot) and the
                     tile-wise combine its question-and-answer part describes.
* ``k1_outer`` / ``rope_angles`` / ``rope_tables`` / ``rope_region``
                  -- the K=1 matmul as one elementwise multiply, the cos /
                     sin tables of its angles, repeated along the last axis,
                     and the query's view / permute / widening steps of the
                     same region ("Schedule a small matmul op as a reduction
                     (or pointwise) op": the %kernel_math listing and the
                     proposed decomposition).
* ``bf16``        -- exact bf16 decode and single-rounding round-to-nearest-
                     even encode.
* ``e4m3_round`` / ``quantize`` / ``gemm_fp8``
                  -- the fp8 cast of "Improve the Inductor generated kernel
                     for the pattern of output1 = pointwise(input); output2 =
                     transpose(output1)" (the example: scale, clamp, cast to
                     e4m3fn) applied to both operands of the GEMM.

Parity pins: every function is pinned in ``tests/test_oracle.py`` against
brute force, closed forms, identities or library routines.  The exact bf16
bits of random-valued GEMM outputs are "parity unpinned" beyond the stated
tolerance, because accumulation order on the GPU differs from BLAS's.
"""

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits
from .gemm import op_matrix, gemm
from .xent import cross_entropy, logsumexp_rows, tile_partials, merge_partials, merge_pair
from .rope import k1_outer, rope_angles, rope_tables, rope_region
from .fp8 import E4M3_MAX, e4m3_round, quantize, gemm_fp8

__all__ = [
    "bf16_bits_to_f64",
    "f64_to_bf16_bits",
    "op_matrix",
    "gemm",
    "cross_entropy",
    "logsumexp_rows",
    "tile_partials",
    "merge_partials",
    "merge_pair",
    "k1_outer",
    "rope_angles",
    "rope_tables",
    "rope_region",
    "E4M3_MAX",
    "e4m3_round",
    "quantize",
    "gemm_fp8",
]
