"""GPU parity of the fp8 (e4m3fn) operand GEMM (tgemm_run_fp8) against the
oracle, through the C-ABI.

Each bf16 operand element is scaled, clamped and cast to e4m3fn; the
products of e4m3fn values are exact, so the only rounding on the GPU is in
the sums and the output scale.  Two routes:
  - cast on load (bf16 matrix cores): held to the fp32 summation bound,
    |error| <= K * 2^-24 * sum |qa qb| (to first order), times the output
    scale, plus one rounding of the product;
  - packed (fp8 matrix cores, v_mfma_f32_32x32x64_f8f6f4): that bound plus
    the matrix core's own group sums.  Measured on MI355X with structured
    inputs: it adds the products of each group of 8 consecutive k at the
    magnitude of the group's largest product, truncating the bits of the
    others below about 2^-12 of it (448 + 7 * 2^-6 gives 448; 65536 + 7 * 1
    gives 65536; groups combine without that loss; subnormal codes are
    exact).  So each group of 8 adds at most 2^-9 * max |qa qb| over the
    group (8 truncated products, each short of one 2^-12 unit).
Integer-valued cases whose group sums stay within that precision are exact
(bitwise) on both routes.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from layout_aware_gemm_amd import tgemm
from parity_util import (FP8_RMS_BF16, FP8_RMS_F32, GEMM_BF16_TOL, bf16_to_f64, bits, dev,
                         fp8_error_bound as error_bound, rms_ratio, scaled_err, within_bound)

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


def takes_packed_route(d, ta, tb, M, N, K):
    """tgemm_run_fp8's packed route: at least two 256-row and two 256-column
    tiles, 16-byte rows (the test tensors are aligned)."""
    colsA = K if ta == "N" else M
    colsB = N if tb == "N" else K
    return (-(-M // 256) >= 2 and -(-N // 256) >= 2 and d["lda"] % 8 == 0
            and d["ldb"] % 8 == 0 and colsA % 8 == 0 and colsB % 8 == 0)


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
    the route's bound, and the bf16 output is the fp32 one rounded once."""
    d = workloads.random_operands(M, N, K, ta, tb, seed=11 * M + N + K, std=30.0)
    scales = (10.0, 0.05, 1.0 / 0.5)
    packed = takes_packed_route(d, ta, tb, M, N, K)
    Cf = run(d, ta, tb, M, N, K, scales).cpu().numpy().astype(np.float64)
    ref = ref_of(d, ta, tb, M, N, K, scales)
    bound = error_bound(d, scales, K, ref, packed=packed)
    assert within_bound(Cf, ref, bound)
    assert rms_ratio(Cf, ref) <= FP8_RMS_F32
    Cb = run(d, ta, tb, M, N, K, scales, out_dtype=torch.bfloat16)
    assert np.array_equal(bits(Cb), oracle.f64_to_bf16_bits(Cf))
    assert within_bound(bf16_to_f64(Cb), ref, bound + np.abs(ref) * 2.0 ** -8)
    if not packed:
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
        bound = error_bound(d2, scales, K, np.nan_to_num(ref))
        assert within_bound(C[ok].astype(np.float64), ref[ok], bound[ok])


# at least two 256-row and two 256-column tiles, every stored row a multiple
# of 8 elements: these take the packed route (a pass casts each operand into
# K-contiguous e4m3fn codes, the fp8 matrix cores multiply them) unless it
# is switched off, which casts on load and multiplies on the bf16 matrix
# cores
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
    """Both routes, every layout, ragged K and ragged tiles (the pack's zero
    padding): integer-valued inputs give the oracle's bits; random inputs,
    unclamped and with op(A) clamping and op(B) reaching subnormals, are
    within the route's bound on sampled rows, and the bf16 output is the
    route's fp32 output rounded once."""
    d = workloads.random_operands(M, N, K, ta, tb, seed=M + N + K, int_range=8)
    assert d["lda"] % 8 == 0 and d["ldb"] % 8 == 0
    scales = (0.5, 2.0, 0.25)
    ref = ref_of(d, ta, tb, M, N, K, scales)
    for route in (1, 0):
        C = run_route(d, ta, tb, M, N, K, scales, route)
        assert np.array_equal(C.cpu().numpy().astype(np.float64), ref)
    rows = [0, 1, M // 2, M - 1]
    for std, scales in ((3.0, (4.0, 8.0, 1.0 / 32)), (30.0, (10.0, 0.05, 2.0))):
        r = workloads.random_operands(M, N, K, ta, tb, seed=M + N + K + int(std), std=std)
        ref = ref_of(r, ta, tb, M, N, K, scales, rows=rows)
        for route in (1, 0):
            bound = error_bound(r, scales, K, ref, rows=rows, packed=route == 1)
            Cf = run_route(r, ta, tb, M, N, K, scales, route)
            assert within_bound(Cf.cpu().numpy()[rows].astype(np.float64), ref, bound)
            assert rms_ratio(Cf.cpu().numpy()[rows], ref) <= FP8_RMS_F32
            Cb = run_route(r, ta, tb, M, N, K, scales, route, out_dtype=torch.bfloat16)
            assert np.array_equal(bits(Cb), oracle.f64_to_bf16_bits(
                Cf.cpu().numpy().astype(np.float64)))


def test_cast_once_keeps_nan():
    """A NaN element survives the pack: its row and column are NaN, like the
    oracle's, and the sampled rows' other entries are within the route's
    bound."""
    M, N, K = 520, 536, 256
    d = workloads.random_operands(M, N, K, "N", "T", seed=41, std=2.0)
    opA, opB = d["opA"].clone(), d["opB"].clone()
    opA[5, 3] = float("nan")
    opB[9, 300] = float("nan")
    sa_, lda = workloads.store_operand(opA, "N")
    sb_, ldb = workloads.store_operand(opB, "T")
    d2 = {"opA": opA, "opB": opB, "A": sa_, "lda": lda, "B": sb_, "ldb": ldb}
    scales = (1.0, 1.0, 1.0)
    for route in (1, 0):
        C = run_route(d2, "N", "T", M, N, K, scales, route)
        nan = torch.isnan(C)
        assert nan[5, :].all() and nan[:, 300].all() and int(nan.sum()) == M + N - 1
        rows = [0, 5, 200, M - 1]
        ref = ref_of(d2, "N", "T", M, N, K, scales, rows=rows)
        got = C.cpu().numpy()[rows].astype(np.float64)
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        ok = ~np.isnan(ref)
        bound = error_bound(d2, scales, K, np.nan_to_num(ref), rows=rows, packed=route == 1)
        assert np.all(np.abs(got - ref)[ok] <= bound[ok])


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_layouts_and_tiles_give_the_same_bits(cfg):
    """The cast happens before the (layout-independent) image the matrix
    cores read -- the packed codes here -- so all four layouts, and every
    tile shape (256x256, 128x128, and the 256x192 the automatic choice
    takes for this shape), give identical bits."""
    M, N, K = 384, 320, 448
    outs = []
    for ta, tb in LAYOUTS:
        d = workloads.random_operands(M, N, K, ta, tb, seed=12, std=20.0)
        outs.append(run(d, ta, tb, M, N, K, (3.0, 7.0, 0.01), cfg=cfg))
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    if cfg != 1:
        d = workloads.random_operands(M, N, K, "N", "T", seed=12, std=20.0)
        assert torch.equal(run(d, "N", "T", M, N, K, (3.0, 7.0, 0.01), cfg=1), outs[0])


@pytest.mark.parametrize("tb", ["T", "N"])
def test_fp8_linear_full_size(tb):
    """The page's float8 linear, 4096x4096 input (scale 10) times a
    [3072, 4096] weight (scale 1000), read in place ('T') or from its
    [4096, 3072] transposed storage ('N') -- the layout the page's pattern
    writes a transposed fp8 copy for.  bf16 output with the inverse scales,
    24 sampled rows against the oracle, within the packed route's bound plus
    one bf16 rounding."""
    w = workloads.fp8_linear()
    M, K, N = 4096, 4096, 3072
    W = w["W"] if tb == "T" else w["W"].t().contiguous()
    d = {"A": w["X"], "lda": K, "B": W, "ldb": K if tb == "T" else N}
    scales = (w["scale_x"], w["scale_w"], 1.0 / (w["scale_x"] * w["scale_w"]))
    C = run(d, "N", tb, M, N, K, scales, out_dtype=torch.bfloat16)
    rows = np.random.default_rng(8).choice(M, 24, replace=False)
    ref = ref_of(d, "N", tb, M, N, K, scales, rows=rows)
    d["opA"] = w["X"]
    d["opB"] = w["W"].t()
    assert takes_packed_route(d, "N", tb, M, N, K)
    bound = error_bound(d, scales, K, ref, rows=rows, packed=True) + np.abs(ref) * 2.0 ** -8
    assert within_bound(bf16_to_f64(C)[rows], ref, bound)
    assert rms_ratio(bf16_to_f64(C)[rows], ref) <= FP8_RMS_BF16
    # and the fp8 product really differs from the bf16 one (the cast happened)
    plain = oracle.gemm("N", tb, M, N, K, workloads.bf16_bits(d["A"]).reshape(-1), d["lda"],
                        workloads.bf16_bits(d["B"]).reshape(-1), d["ldb"], rows=rows)
    assert np.max(np.abs(ref - plain)) > 1e-3
