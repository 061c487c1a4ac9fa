"""GPU parity of the fp8 (e4m3fn) operand GEMM (tgemm_run_fp8) against the
oracle, through the C-ABI.

Each bf16 operand element is scaled, clamped and cast to e4m3fn as the
kernel loads it; the products of e4m3fn values are exact, so the only
rounding on the GPU is the fp32 accumulation and the output scale.
Integer-valued cases are therefore exact (bitwise), and random cases are
held to the fp32 summation bound: |error| <= K * 2^-24 * sum |qa qb| (to
first order), times the output scale, plus one rounding of the product.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from layout_aware_gemm_amd import tgemm
from parity_util import GEMM_BF16_TOL, bf16_to_f64, bits, dev, scaled_err

pytestmark = pytest.mark.gpu

LAYOUTS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]


def run(d, ta, tb, M, N, K, scales, out_dtype=torch.float32, ldc=None, cfg=0):
    A, B = d["A"].to(dev()), d["B"].to(dev())
    ldc = N if ldc is None else ldc
    C = torch.full((M, ldc), float("nan"), dtype=out_dtype, device=dev())
    sc = torch.tensor(scales, dtype=torch.float32, device=dev())
    epi = tgemm.EPI_STORE_BF16 if out_dtype == torch.bfloat16 else tgemm.EPI_STORE_F32
    prev = tgemm.set_tile_config(cfg)
    try:
        tgemm.run_fp8(ta, tb, M, N, K, A, d["lda"], B, d["ldb"], C, ldc, epi, sc)
        torch.cuda.synchronize()
    finally:
        tgemm.set_tile_config(prev)
    return C


def ref_of(d, ta, tb, M, N, K, scales, rows=None):
    return oracle.gemm_fp8(ta, tb, M, N, K, workloads.bf16_bits(d["A"]).reshape(-1), d["lda"],
                           workloads.bf16_bits(d["B"]).reshape(-1), d["ldb"], *scales, rows=rows)


def abs_products(d, ta, tb, M, N, K, scales, rows=None):
    """out_scale * sum_k |qa qb| in fp64 (the summation bound)."""
    sa, sb, so = scales
    qa = np.abs(oracle.quantize(d["opA"].float().numpy(), sa))
    qb = np.abs(oracle.quantize(d["opB"].float().numpy(), sb))
    if rows is not None:
        qa = qa[np.asarray(rows)]
    return (qa @ qb) * abs(so)


def within_f32_bound(C, ref, absprod, K):
    bound = K * 2.0 ** -24 * absprod * 1.01 + np.abs(ref) * 2.0 ** -23 + 1e-30
    return np.all(np.abs(C - ref) <= bound)


SHAPES = [(64, 48, 64), (300, 260, 200), (257, 129, 100), (1, 50, 70), (40, 1, 33), (33, 17, 1),
          (520, 530, 136)]


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_integer_valued_is_exact(M, N, K, ta, tb):
    """Integers in [-8, 8]: the casts are exact (x 0.5 and x 2 keep them on
    the e4m3fn grid), every partial sum is exact in fp32, the output scale
    is a power of two: the result equals the oracle bit for bit, and nothing
    is written past column N."""
    d = workloads.random_operands(M, N, K, ta, tb, seed=M + 3 * N + 7 * K, pad=3, int_range=8)
    for scales in [(1.0, 1.0, 0.25), (0.5, 2.0, 1.0)]:
        C = run(d, ta, tb, M, N, K, scales, ldc=N + 2)
        ref = ref_of(d, ta, tb, M, N, K, scales)
        assert np.array_equal(C[:, :N].cpu().numpy().astype(np.float64), ref)
        assert torch.isnan(C[:, N:]).all()


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(300, 260, 200), (257, 129, 1000), (64, 64, 4096)])
def test_scale_clamp_round_against_oracle(M, N, K, ta, tb):
    """N(0, 30) inputs times 10 and 0.05: most of op(A) clamps to +-448, op(B)
    lands on the whole e4m3fn range including subnormals; fp32 output within
    the summation bound, and the bf16 output is the fp32 one rounded once."""
    d = workloads.random_operands(M, N, K, ta, tb, seed=11 * M + N + K, std=30.0)
    scales = (10.0, 0.05, 1.0 / 0.5)
    Cf = run(d, ta, tb, M, N, K, scales).cpu().numpy().astype(np.float64)
    ref = ref_of(d, ta, tb, M, N, K, scales)
    assert within_f32_bound(Cf, ref, abs_products(d, ta, tb, M, N, K, scales), K)
    Cb = run(d, ta, tb, M, N, K, scales, out_dtype=torch.bfloat16)
    assert np.array_equal(bits(Cb), oracle.f64_to_bf16_bits(Cf))
    assert scaled_err(bf16_to_f64(Cb), ref) <= GEMM_BF16_TOL


def test_nan_propagates_through_the_cast():
    """A NaN input element stays NaN through scale and clamp (it does not
    clamp to 448): its output row (from A) and column (from B) are NaN,
    everything else matches the oracle."""
    M, N, K = 200, 180, 150
    for ta, tb in LAYOUTS:
        d = workloads.random_operands(M, N, K, ta, tb, seed=5, std=2.0)
        opA, opB = d["opA"].clone(), d["opB"].clone()
        opA[7, 33] = float("nan")
        opB[90, 101] = float("nan")
        sa_, lda = workloads.store_operand(opA, ta)
        sb_, ldb = workloads.store_operand(opB, tb)
        d2 = {"opA": opA, "opB": opB, "A": sa_, "lda": lda, "B": sb_, "ldb": ldb}
        scales = (1.0, 1.0, 1.0)
        C = run(d2, ta, tb, M, N, K, scales).cpu().numpy()
        nan = np.isnan(C)
        assert nan[7, :].all() and nan[:, 101].all()
        assert nan.sum() == N + M - 1
        ref = ref_of(d2, ta, tb, M, N, K, scales)
        ok = ~nan
        absprod = abs_products(d2, ta, tb, M, N, K, scales)
        assert within_f32_bound(C[ok].astype(np.float64), ref[ok], absprod[ok], K)


# at least two 256-row and two 256-column tiles, every stored row a multiple
# of 8 elements: these take the cast-once route (a cast pass into a compact
# copy, then the GEMM on plain bf16) unless it is switched off
CAST_ONCE = [(600, 520, 1000), (520, 536, 136), (1024, 768, 512)]


def run_route(d, ta, tb, M, N, K, scales, cast_once, **kw):
    prev = tgemm.set_fp8_cast_once(cast_once)
    try:
        return run(d, ta, tb, M, N, K, scales, **kw)
    finally:
        tgemm.set_fp8_cast_once(prev)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", CAST_ONCE)
def test_cast_once_route(M, N, K, ta, tb):
    """Integer-valued inputs: the oracle's bits.  Random inputs: the same
    bits as casting on load, in fp32 and bf16, and within the fp32 bound."""
    d = workloads.random_operands(M, N, K, ta, tb, seed=M + N + K, int_range=8)
    assert d["lda"] % 8 == 0 and d["ldb"] % 8 == 0
    scales = (0.5, 2.0, 0.25)
    C = run_route(d, ta, tb, M, N, K, scales, 1)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), ref_of(d, ta, tb, M, N, K, scales))
    r = workloads.random_operands(M, N, K, ta, tb, seed=M + N + K + 1, std=3.0)
    scales = (4.0, 8.0, 1.0 / 32)
    for dt in (torch.float32, torch.bfloat16):
        once = run_route(r, ta, tb, M, N, K, scales, 1, out_dtype=dt)
        load = run_route(r, ta, tb, M, N, K, scales, 0, out_dtype=dt)
        if dt == torch.bfloat16:
            assert np.array_equal(bits(once), bits(load))
        else:
            assert torch.equal(once, load)
    rows = [0, 1, M // 2, M - 1]
    once_f32 = run_route(r, ta, tb, M, N, K, scales, 1)
    ref = ref_of(r, ta, tb, M, N, K, scales, rows=rows)
    absprod = abs_products(r, ta, tb, M, N, K, scales, rows=rows)
    assert within_f32_bound(once_f32.cpu().numpy()[rows].astype(np.float64), ref, absprod, K)


def test_cast_once_keeps_nan():
    """A NaN element survives the cast pass: its row and column are NaN, the
    rest equals the cast-on-load route bit for bit."""
    M, N, K = 520, 536, 256
    d = workloads.random_operands(M, N, K, "N", "T", seed=41, std=2.0)
    opA, opB = d["opA"].clone(), d["opB"].clone()
    opA[5, 3] = float("nan")
    opB[9, 300] = float("nan")
    sa_, lda = workloads.store_operand(opA, "N")
    sb_, ldb = workloads.store_operand(opB, "T")
    d2 = {"opA": opA, "opB": opB, "A": sa_, "lda": lda, "B": sb_, "ldb": ldb}
    once = run_route(d2, "N", "T", M, N, K, (1.0, 1.0, 1.0), 1)
    load = run_route(d2, "N", "T", M, N, K, (1.0, 1.0, 1.0), 0)
    nan = torch.isnan(once)
    assert nan[5, :].all() and nan[:, 300].all() and int(nan.sum()) == M + N - 1
    assert torch.equal(torch.isnan(load), nan)
    assert torch.equal(once[~nan], load[~nan])


@pytest.mark.parametrize("cfg", [1, 2])
def test_layouts_and_tiles_give_the_same_bits(cfg):
    """The cast happens before the (layout-independent) LDS image, so all
    four layouts, and both tile configurations, give identical bits."""
    M, N, K = 384, 320, 448
    outs = []
    for ta, tb in LAYOUTS:
        d = workloads.random_operands(M, N, K, ta, tb, seed=12, std=20.0)
        outs.append(run(d, ta, tb, M, N, K, (3.0, 7.0, 0.01), cfg=cfg))
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    if cfg == 2:
        d = workloads.random_operands(M, N, K, "N", "T", seed=12, std=20.0)
        assert torch.equal(run(d, "N", "T", M, N, K, (3.0, 7.0, 0.01), cfg=1), outs[0])


@pytest.mark.parametrize("tb", ["T", "N"])
def test_fp8_linear_full_size(tb):
    """The page's float8 linear, 4096x4096 input (scale 10) times a
    [3072, 4096] weight (scale 1000), read in place ('T') or from its
    [4096, 3072] transposed storage ('N') -- the layout the page's pattern
    writes a transposed fp8 copy for.  bf16 output with the inverse scales,
    24 sampled rows against the oracle."""
    w = workloads.fp8_linear()
    M, K, N = 4096, 4096, 3072
    W = w["W"] if tb == "T" else w["W"].t().contiguous()
    d = {"A": w["X"], "lda": K, "B": W, "ldb": K if tb == "T" else N}
    scales = (w["scale_x"], w["scale_w"], 1.0 / (w["scale_x"] * w["scale_w"]))
    C = run(d, "N", tb, M, N, K, scales, out_dtype=torch.bfloat16)
    rows = np.random.default_rng(8).choice(M, 24, replace=False)
    ref = ref_of(d, "N", tb, M, N, K, scales, rows=rows)
    assert scaled_err(bf16_to_f64(C)[rows], ref) <= GEMM_BF16_TOL
    # and the fp8 product really differs from the bf16 one (the cast happened)
    plain = oracle.gemm("N", tb, M, N, K, workloads.bf16_bits(d["A"]).reshape(-1), d["lda"],
                        workloads.bf16_bits(d["B"]).reshape(-1), d["ldb"], rows=rows)
    assert np.max(np.abs(ref - plain)) > 1e-3
