"""bf16 <-> fp64 for the oracle (test infrastructure only).

The pages cast fp32 results to a 16-bit float without naming a rounding mode
("Schedule a small matmul op ...", %kernel_math: the final float-to-bfloat
cast; "Allow reductions in matmul epilogues": the cast of the softmax-minus-
one-hot matrix).  The reading taken here is IEEE round-to-nearest-even, NaN
kept as a quiet NaN, subnormals kept.

Encoding works from the fp64 value with ONE rounding (no detour through
fp32), so a value computed in fp64 by the oracle is rounded exactly once.
"""

import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_QNAN_BITS = 0x7FC0


def bf16_bits_to_f64(bits):
    """Decode bf16 bit patterns (any integer array of 16-bit values) to fp64.

    bf16 is the top half of an IEEE binary32, so the decode is exact:
    shift the 16 bits into the high half of a 32-bit word, read it as
    binary32 and widen to binary64.
    """
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round fp64 values to bf16 (round-to-nearest, ties-to-even); uint16 bits.

    A bf16 normal number has 8 significant bits, so in the binade
    [2**(e-1), 2**e) its spacing is 2**(e-8); below the smallest normal
    (2**-126) the spacing is fixed at 2**-133.  The magnitude is divided by
    its spacing, rounded to an integer with ties to even (``np.rint``) and
    scaled back, which lands exactly on the bf16 grid (also when rounding
    carries into the next binade).  Results above the largest finite bf16
    become infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                       # a = f * 2**e, 0.5 <= f < 1
    spacing_exp = np.maximum(e - 8, -133)
    with np.errstate(over="ignore", invalid="ignore"):
        q = np.rint(np.ldexp(a, -spacing_exp))
        r = np.ldexp(q, spacing_exp)
    r = np.where(r > _BF16_MAX, np.inf, r)
    r = np.where(np.isinf(a), np.inf, r)
    r = np.where(np.signbit(x), -r, r)
    with np.errstate(invalid="ignore"):
        bits = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(_QNAN_BITS), bits).astype(np.uint16)
    return bits
