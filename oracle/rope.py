"""Oracle for the degenerate K=1 matmul and its RoPE epilogue (test infra only).

Follows "Schedule a small matmul op as a reduction (or pointwise) op":

* the %kernel_math listing: the [64] inverse frequencies widened to fp32 and
  broadcast to [1, 64, 1]; the int64 positions [1, 4096] cast to fp32 and
  broadcast to [1, 1, 4096]; their K=1 matmul giving fp32 [1, 64, 4096];
  a permute to [1, 4096, 64]; two pads and a cat that duplicate the last
  dimension to 128; cos; a cast to bf16;
* the proposed decomposition: that K=1 matmul is a broadcast, an elementwise
  multiply and a squeeze, i.e. one fp32 multiply per output element.

Readings: the pad/pad/cat pair is read as cat(T, T) along the last dimension
(emb[p, d] = T[p, d mod 64]); the second declared [1, 1, 4096, 128] bf16
output, whose math the listing cuts off, is read as the sin twin of the cos
output; the inverse frequencies are taken as fp32 inputs.
"""

import numpy as np

from .bf16 import f64_to_bf16_bits


def k1_outer(a_f32, b_f32):
    """K=1 product t[i, j] = a[i] * b[j], each element rounded once to fp32.

    The two fp32 factors have 24-bit significands, so their fp64 product is
    exact and a single rounding to fp32 gives the IEEE fp32 product.
    """
    a = np.asarray(a_f32, dtype=np.float32).astype(np.float64)
    b = np.asarray(b_f32, dtype=np.float32).astype(np.float64)
    return (a[:, None] * b[None, :]).astype(np.float32)


def rope_tables(pos_i64, inv_freq_f32):
    """Return (T19 fp32 [N, P], emb fp32 [P, 2N], cos bf16 bits, sin bf16 bits).

    N = len(inv_freq), P = len(pos).  cos and sin are [P, 2N] uint16 arrays,
    each the fp64 cos/sin of the fp32 table value rounded once to bf16.
    """
    pos = np.asarray(pos_i64, dtype=np.int64).reshape(-1)
    inv_freq = np.asarray(inv_freq_f32, dtype=np.float32).reshape(-1)
    pos32 = pos.astype(np.float32)                 # int64 -> fp32 cast
    t19 = k1_outer(inv_freq, pos32)                # [N, P], the page's order
    t20 = np.ascontiguousarray(t19.T)              # permute -> [P, N]
    emb = np.concatenate([t20, t20], axis=1)       # duplicate -> [P, 2N]
    e64 = emb.astype(np.float64)
    cos_bits = f64_to_bf16_bits(np.cos(e64))
    sin_bits = f64_to_bf16_bits(np.sin(e64))
    return t19, emb, cos_bits, sin_bits
