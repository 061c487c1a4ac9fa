"""GPU parity of the matrix-vector and dot-product path (M = 1 or N = 1,
K > 1), through the C-ABI, against the oracle.

Integer-valued inputs make the fp32 result exact in any summation order
(every partial sum is an integer below 2^24), so those cases compare bit
for bit and catch a dropped or repeated K chunk.  Random inputs are held to
the bf16 rule, and fp32 outputs to the bound for any order of summing K
products in fp32: |error| <= K * 2^-24 * sum |a_k b_k| (to first order).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from layout_aware_gemm_amd import tgemm
from parity_util import GEMM_BF16_TOL, bf16_to_f64, bits, dev, oracle_gemm_from, scaled_err

pytestmark = pytest.mark.gpu

LAYOUTS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]


def run(d, ta, tb, M, N, K, out_dtype, ldc=None):
    A, B = d["A"].to(dev()), d["B"].to(dev())
    ldc = N if ldc is None else ldc
    C = torch.full((M, ldc), float("nan"), dtype=out_dtype, device=dev())
    epi = tgemm.EPI_STORE_BF16 if out_dtype == torch.bfloat16 else tgemm.EPI_STORE_F32
    tgemm.run(ta, tb, M, N, K, A, d["lda"], B, d["ldb"], C, ldc, epi)
    torch.cuda.synchronize()
    return C


def abs_products(d):
    """sum over k of |op(A)[m,k] op(B)[k,n]| in fp64 (the summation bound)."""
    return (d["opA"].double().abs() @ d["opB"].double().abs()).numpy()


SHAPES = [(1, 1, 2), (1, 1, 513), (1, 1, 70001), (1, 7, 100), (1, 300, 4097), (1, 2049, 1000),
          (1, 5000, 777), (5, 1, 9000), (300, 1, 4097), (2049, 1, 513), (4100, 1, 64)]


@pytest.mark.parametrize("pad", [0, 3])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_integer_valued_is_exact(M, N, K, ta, tb, pad):
    d = workloads.random_operands(M, N, K, ta, tb, seed=M * 3 + N * 5 + K, pad=pad, int_range=4)
    C = run(d, ta, tb, M, N, K, torch.float32, ldc=N + 2)
    ref = oracle_gemm_from(d, ta, tb, M, N, K)
    assert np.array_equal(C[:, :N].cpu().numpy().astype(np.float64), ref)
    assert torch.isnan(C[:, N:]).all()           # nothing written past N


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_random_bf16_and_f32(M, N, K, ta, tb):
    d = workloads.random_operands(M, N, K, ta, tb, seed=M + N * 7 + K * 3)
    ref = oracle_gemm_from(d, ta, tb, M, N, K)
    Cb = run(d, ta, tb, M, N, K, torch.bfloat16)
    assert scaled_err(bf16_to_f64(Cb), ref) <= GEMM_BF16_TOL
    Cf = run(d, ta, tb, M, N, K, torch.float32).cpu().numpy().astype(np.float64)
    bound = K * 2.0 ** -24 * abs_products(d) * 1.01 + 1e-30
    assert np.all(np.abs(Cf - ref) <= bound)
    # the bf16 result is the fp32 result rounded once
    assert np.array_equal(bits(Cb), oracle.f64_to_bf16_bits(Cf))


def test_repeat_calls_same_bits():
    M, N, K = 1, 5120, 13824
    d = workloads.random_operands(M, N, K, "N", "T", seed=3)
    outs = [run(d, "N", "T", M, N, K, torch.float32) for _ in range(3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("tb", ["T", "N"])
def test_decode_step_gemv_full_size(tb):
    """x[1, 13824] . W: the down-projection for one token, W [5120, 13824]
    read in place ('T', rows of K) or a [13824, 5120] weight ('N')."""
    w = workloads.nt_mlp()
    x = w["X"].reshape(-1, 13824)[:1].contiguous()
    W = w["W"] if tb == "T" else w["W"].t().contiguous()
    d = {"A": x, "lda": 13824, "B": W, "ldb": 13824 if tb == "T" else 5120}
    C = run(d, "N", tb, 1, 5120, 13824, torch.bfloat16)
    ref = oracle_gemm_from(d, "N", tb, 1, 5120, 13824)
    assert scaled_err(bf16_to_f64(C), ref) <= GEMM_BF16_TOL


def test_long_dot_exact():
    """A dot product of 2^24 - 1 values in {-1, 0, 1}: every partial sum is an
    integer of magnitude below 2^24, so the fp32 result is exact."""
    K = 2 ** 24 - 1
    g = torch.Generator().manual_seed(11)
    a = torch.randint(-1, 2, (K,), generator=g).to(torch.bfloat16)
    b = torch.randint(-1, 2, (K,), generator=g).to(torch.bfloat16)
    C = torch.empty(1, 1, dtype=torch.float32, device=dev())
    tgemm.run("N", "N", 1, 1, K, a.to(dev()), K, b.to(dev()), 1, C, 1, tgemm.EPI_STORE_F32)
    ref = oracle.gemm("N", "N", 1, 1, K, workloads.bf16_bits(a), K, workloads.bf16_bits(b), 1)
    assert C.item() == ref[0, 0]
