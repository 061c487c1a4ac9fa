"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This module only draws and lays out inputs; it holds none of the method's
arithmetic, and it imports neither the oracle nor the HIP binding.  Every
tensor is a CPU tensor; callers copy it to the device themselves.  Random
values come from a CPU ``torch.Generator`` seeded per workload, drawn as fp32
``randn`` (scaled as stated) and cast to bf16 with round-to-nearest-even.

Workloads (shapes and distributions of the pages' examples):

* ``tiny_ce``      A bf16[64,128], W bf16[256,128], both N(0,1)/sqrt(128),
                   labels int32[64] uniform in [0, 256)              seed 1001
* ``nt_mlp``       X bf16[384,2,13824] N(0,1) (viewed [768,13824]),
                   W bf16[5120,13824] N(0,0.02) -- the down-projection of
                   "Strength reduction: fold transpose into a subsequent
                   GEMM call" (the trace's shapes)                   seed 1002
* ``layout_sweep`` logical op(A), op(B) bf16[4096,4096] N(0,1)/64, stored in
                   each of the four layouts                          seed 1003
* ``ce_vocab``     H bf16[4096,4096] N(0,1), W bf16[32000,4096] N(0,0.02),
                   labels int32[4096] uniform in [0, 32000)          seed 1004
* ``rope``         inv_freq fp32[64] = 10000**(-2i/128) (fp64, rounded once),
                   positions int64[4096] = 0..4095 -- the RoPE region of
                   "Schedule a small matmul op as a reduction (or pointwise)
                   op" (its fusion inputs)                          deterministic
* ``rope_batched`` the same table for ``batch`` sequences of 0..4095
* ``rope_region``  the same positions and frequencies with the region's
                   query bf16[4096, 32*128] N(0,1) (the listing's T0) seed 1006
* ``fp8_linear``   X bf16[4096,4096] N(0,1), W bf16[3072,4096] N(0,0.02) with
                   the cast scales {10, 1000} -- the float8 linear of "Improve
                   the Inductor generated kernel for the pattern of output1 =
                   pointwise(input); output2 = transpose(output1)" (the
                   example's M, K, N = 4096, 4096, 3072 and its input scale
                   10; the weight's scale puts its values in the e4m3fn
                   range the same way)                               seed 1005
"""

import math

import numpy as np
import torch

SEEDS = {"tiny_ce": 1001, "nt_mlp": 1002, "layout_sweep": 1003, "ce_vocab": 1004,
         "rope_region": 1006,
         "fp8_linear": 1005}


def _gen(seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def randn_bf16(shape, std, gen):
    """fp32 N(0, std^2) draws cast to bf16 (round-to-nearest-even)."""
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def bf16_bits(t):
    """CPU bf16 tensor -> NumPy uint16 bit patterns (same bytes, no copy)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def store_operand(logical, trans):
    """Lay out a logical [R, C] operand in memory for a layout letter.

    For op(A) = logical [M, K]: 'N' stores [M, K], 'T' stores [K, M].
    For op(B) = logical [K, N]: 'N' stores [K, N], 'T' stores [N, K].
    Returns a contiguous tensor (the stored array) and its leading dimension.
    """
    if trans == "N":
        s = logical.contiguous()
    elif trans == "T":
        s = logical.t().contiguous()
    else:
        raise ValueError(trans)
    return s, s.shape[1]


def tiny_ce(seed=SEEDS["tiny_ce"]):
    g = _gen(seed)
    a = randn_bf16((64, 128), 1.0 / math.sqrt(128.0), g)
    w = randn_bf16((256, 128), 1.0 / math.sqrt(128.0), g)
    labels = torch.randint(0, 256, (64,), generator=g, dtype=torch.int32)
    return {"A": a, "W": w, "labels": labels}


def nt_mlp(seed=SEEDS["nt_mlp"], batch=384, pairs=2, hidden=13824, out=5120):
    g = _gen(seed)
    x = randn_bf16((batch, pairs, hidden), 1.0, g)
    w = randn_bf16((out, hidden), 0.02, g)
    return {"X": x, "W": w}


def layout_sweep(seed=SEEDS["layout_sweep"], M=4096, N=4096, K=4096):
    """Logical op(A) [M, K] and op(B) [K, N]; store with ``store_operand``."""
    g = _gen(seed)
    a = randn_bf16((M, K), 1.0 / 64.0, g)
    b = randn_bf16((K, N), 1.0 / 64.0, g)
    return {"opA": a, "opB": b}


def ce_vocab(seed=SEEDS["ce_vocab"], M=4096, N=32000, K=4096):
    g = _gen(seed)
    h = randn_bf16((M, K), 1.0, g)
    w = randn_bf16((N, K), 0.02, g)
    labels = torch.randint(0, N, (M,), generator=g, dtype=torch.int32)
    return {"H": h, "W": w, "labels": labels}


def inv_freq(dim=128, base=10000.0):
    """fp32[dim/2] inverse frequencies base**(-2i/dim), fp64 then one rounding."""
    i = np.arange(dim // 2, dtype=np.float64)
    return torch.from_numpy((base ** (-(2.0 * i) / dim)).astype(np.float32))


def rope(seq=4096, dim=128):
    return {"pos": torch.arange(seq, dtype=torch.int64), "inv_freq": inv_freq(dim)}


def rope_region(seed=SEEDS["rope_region"], seq=4096, heads=32, dim=128):
    """The region's inputs: the query bf16 [seq, heads*dim] N(0,1) (the
    listing's T0, [1, 4096, 4096]), positions 0..seq-1 and the inverse
    frequencies of ``rope``."""
    g = _gen(seed)
    return {"q": randn_bf16((seq, heads * dim), 1.0, g), "heads": heads,
            "pos": torch.arange(seq, dtype=torch.int64), "inv_freq": inv_freq(dim)}


def rope_batched(batch=256, seq=4096, dim=128):
    pos = torch.arange(seq, dtype=torch.int64).repeat(batch)
    return {"pos": pos, "inv_freq": inv_freq(dim)}


def fp8_linear(seed=SEEDS["fp8_linear"], M=4096, K=4096, N=3072):
    g = _gen(seed)
    x = randn_bf16((M, K), 1.0, g)
    w = randn_bf16((N, K), 0.02, g)
    return {"X": x, "W": w, "scale_x": 10.0, "scale_w": 1000.0}


def random_operands(M, N, K, transA, transB, seed, std=1.0, pad=0, int_range=None):
    """Small/ragged cases: logical op(A), op(B) and their stored forms.

    ``pad`` adds that many unused columns to each stored row (ld > minimum).
    ``int_range`` = r draws integers in [-r, r] instead of normals.
    """
    g = _gen(seed)
    if int_range is None:
        a = randn_bf16((M, K), std, g)
        b = randn_bf16((K, N), std, g)
    else:
        a = torch.randint(-int_range, int_range + 1, (M, K), generator=g).to(torch.bfloat16)
        b = torch.randint(-int_range, int_range + 1, (K, N), generator=g).to(torch.bfloat16)
    sa, lda = store_operand(a, transA)
    sb, ldb = store_operand(b, transB)
    if pad:
        sa = torch.cat([sa, torch.zeros(sa.shape[0], pad, dtype=sa.dtype)], 1).contiguous()
        sb = torch.cat([sb, torch.zeros(sb.shape[0], pad, dtype=sb.dtype)], 1).contiguous()
        lda += pad
        ldb += pad
    return {"opA": a, "opB": b, "A": sa, "lda": lda, "B": sb, "ldb": ldb}
