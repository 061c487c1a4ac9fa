"""Oracle for the degenerate K=1 matmul and its RoPE epilogue (test infra only).

What is computed ("Schedule a small matmul op as a reduction (or pointwise)
op": the fusion's inputs and outputs, the %kernel_math listing and the
proposed decomposition of its K = 1 matmul): the angle of position p and
frequency i is the fp32 product of the position cast to fp32 and the
inverse frequency,

    angle[p, i] = fp32(fp32(pos[p]) * inv_freq[i]),

a K = 1 matmul, i.e. one elementwise multiply of two broadcast operands.
The tables the region emits are cos and sin of those angles, rounded to
bf16, with the F frequencies repeated once along the last axis:

    cos_table[p, d] = bf16(cos(angle[p, d mod F])),  d < 2F,  likewise sin.

Readings: the two pads and the cat of the listing are read as the last axis
written twice (table column d holds frequency d mod F); the second declared
bf16 [4096, 128] output, whose math the listing cuts off after cos, is read
as the sin table; the inverse frequencies are taken as fp32 inputs.  The
page multiplies in the order [frequencies] x [positions] and then permutes;
an fp32 product is exactly rounded and commutes, so the [positions,
frequencies] product here has the same bits (a pin checks this).
"""

import numpy as np

from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits


def k1_outer(a_f32, b_f32):
    """K=1 product t[i, j] = a[i] * b[j], each element rounded once to fp32.

    The two fp32 factors have 24-bit significands, so their fp64 product is
    exact and a single rounding to fp32 gives the IEEE fp32 product.
    """
    a = np.asarray(a_f32, dtype=np.float32).astype(np.float64)
    b = np.asarray(b_f32, dtype=np.float32).astype(np.float64)
    return (a[:, None] * b[None, :]).astype(np.float32)


def rope_angles(pos_i64, inv_freq_f32):
    """fp32 angles [P, F]: the position (int64 cast to fp32) times each
    inverse frequency."""
    pos32 = np.asarray(pos_i64, dtype=np.int64).reshape(-1).astype(np.float32)
    return k1_outer(pos32, np.asarray(inv_freq_f32, dtype=np.float32).reshape(-1))


def rope_tables(pos_i64, inv_freq_f32):
    """Return (angles fp32 [P, F], cos bf16 bits [P, 2F], sin bf16 bits [P, 2F]).

    Each table entry is the fp64 cos / sin of the fp32 angle, rounded once to
    bf16; column d uses frequency d mod F.
    """
    angles = rope_angles(pos_i64, inv_freq_f32)
    wide = np.hstack([angles, angles]).astype(np.float64)
    return angles, f64_to_bf16_bits(np.cos(wide)), f64_to_bf16_bits(np.sin(wide))


def rope_region(q_bits, ldq, P, H, D, pos_i64, inv_freq_f32):
    """The region's query steps and tables, as far as the listing goes.

    The query rows (bf16 bits, P rows of stride ldq, H heads of D values per
    row) are viewed as [P, H, D], permuted to [H, P, D] and widened from bf16
    (exact); the tables are ``rope_tables`` of the positions with the D/2
    inverse frequencies.  Returns (q_heads fp64 [H, P, D], angles, cos bits,
    sin bits).  The rotation that would combine them is not on the page.
    """
    flat = np.asarray(q_bits).reshape(-1)
    if flat.size < (P - 1) * ldq + H * D or ldq < H * D:
        raise ValueError("query buffer too small for its shape and row stride")
    rows = np.stack([flat[p * ldq: p * ldq + H * D] for p in range(P)])     # [P, H*D]
    as_heads = rows.reshape(P, H, D)                                         # view
    head_major = np.ascontiguousarray(as_heads.transpose(1, 0, 2))          # permute
    q_heads = bf16_bits_to_f64(head_major)                                   # widen
    angles, cos_bits, sin_bits = rope_tables(pos_i64, inv_freq_f32)
    if cos_bits.shape[1] != D:
        raise ValueError("the tables are D = 2 * len(inv_freq) wide")
    return q_heads, angles, cos_bits, sin_bits
