"""GPU parity of the layout-aware GEMM (store epilogues) against the oracle.

Every call goes through the C-ABI (``tgemm.run``).  Inputs are seeded and
identical on both sides; expected values come only from ``oracle``.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from layout_aware_gemm_amd import tgemm
from parity_util import (GEMM_BF16_TOL, GEMM_REL_TOL, bf16_to_f64, bits, dev, oracle_gemm_from,
                         rms_rel_err, sample_rows, scaled_err)

pytestmark = pytest.mark.gpu

LAYOUTS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]
RAGGED = [(1, 1, 1), (3, 7, 13), (33, 65, 257), (257, 129, 65), (300, 333, 200),
          (129, 257, 1000), (64, 256, 128), (520, 136, 72)]


def run_store(d, ta, tb, M, N, K, out_dtype=torch.bfloat16, cfg=0, ldc=None):
    A = d["A"].to(dev())
    B = d["B"].to(dev())
    ldc = N if ldc is None else ldc
    C = torch.full((M, ldc), float("nan"), dtype=out_dtype, device=dev())
    epi = tgemm.EPI_STORE_BF16 if out_dtype == torch.bfloat16 else tgemm.EPI_STORE_F32
    prev = tgemm.set_tile_config(cfg)
    try:
        tgemm.run(ta, tb, M, N, K, A, d["lda"], B, d["ldb"], C, ldc, epi)
    finally:
        tgemm.set_tile_config(prev)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("cfg", [1, 2, 3])
@pytest.mark.parametrize("pad", [0, 3])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", RAGGED)
def test_ragged_bf16(M, N, K, ta, tb, pad, cfg):
    d = workloads.random_operands(M, N, K, ta, tb, seed=M * 7 + N * 3 + K, pad=pad)
    C = run_store(d, ta, tb, M, N, K, cfg=cfg, ldc=N + 5)
    ref = oracle_gemm_from(d, ta, tb, M, N, K)
    got = bf16_to_f64(C[:, :N])
    assert scaled_err(got, ref) <= GEMM_BF16_TOL
    assert torch.isnan(C[:, N:].float()).all()          # nothing written past N


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(96, 80, 1024), (257, 300, 520), (1000, 64, 999)])
def test_integer_valued_is_exact(M, N, K, ta, tb):
    # entries in {-4..4}, K <= 1024: every partial sum is an integer below
    # 2^24, so fp32 accumulation is exact in any order -> bitwise equality
    d = workloads.random_operands(M, N, K, ta, tb, seed=K, int_range=4)
    C = run_store(d, ta, tb, M, N, K, out_dtype=torch.float32)
    ref = oracle_gemm_from(d, ta, tb, M, N, K)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("K", [320, 384, 64, 4096 - 64])
def test_interior_256_tiles_odd_and_even_k_steps(K, ta, tb):
    """Whole 256x256 tiles in every layout with an odd (5, 1, 63) and an
    even (6) count of 64-wide k-steps: the direct-copy, mixed and two-set
    loops peel k-step 0 when the count is odd.  Integer entries: the
    oracle's bits, in fp32 and bf16 output."""
    M, N = 512, 768
    d = workloads.random_operands(M, N, K, ta, tb, seed=K + 5, int_range=3)
    ref = oracle_gemm_from(d, ta, tb, M, N, K)
    C = run_store(d, ta, tb, M, N, K, out_dtype=torch.float32, cfg=1)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), ref)
    Cb = run_store(d, ta, tb, M, N, K, cfg=1)
    assert np.array_equal(bits(Cb), oracle.f64_to_bf16_bits(ref))


def test_integer_valued_bf16_output_is_exact():
    # |C| <= 256 keeps every integer exactly representable in bf16
    M, N, K = 200, 136, 16
    d = workloads.random_operands(M, N, K, "N", "T", seed=77, int_range=4)
    C = run_store(d, "N", "T", M, N, K)
    ref = oracle_gemm_from(d, "N", "T", M, N, K)
    assert np.abs(ref).max() <= 256
    assert np.array_equal(bits(C), oracle.f64_to_bf16_bits(ref))


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_layouts_bitwise_identical(cfg):
    M, N, K = 384, 320, 448
    outs = []
    for ta, tb in LAYOUTS:
        d = workloads.random_operands(M, N, K, ta, tb, seed=12)
        outs.append(run_store(d, ta, tb, M, N, K, out_dtype=torch.float32, cfg=cfg))
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


@pytest.mark.parametrize("M,N,K", [(300, 260, 200), (512, 768, 640)])
def test_tile_configs_agree(M, N, K):
    # the 256x256, 128x128 and 192x256 tile kernels (interior tiles on the
    # global->LDS path, edge tiles on the register path) must produce the
    # same bits
    d = workloads.random_operands(M, N, K, "N", "T", seed=13)
    outs = [run_store(d, "N", "T", M, N, K, out_dtype=torch.float32, cfg=c) for c in (1, 2, 3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def _spread_rows(X, ld):
    """X [rows, cols] copied into device memory with row stride ``ld``
    elements (only the first ``cols`` of each stride are written or read)."""
    rows, cols = X.shape
    flat = torch.empty((rows - 1) * ld + cols, dtype=X.dtype, device=dev())
    view = flat.as_strided((rows, cols), (ld, 1))
    view.copy_(X.to(dev()))
    return view


@pytest.mark.parametrize("ta,tb", [("N", "T"), ("T", "N")])
def test_leading_dimension_past_2_pow_23(ta, tb):
    # row strides of 2^23 + 64 elements (16 MiB rows, 2-5 GB per operand):
    # the tiles leave the 32-bit-offset buffer loads for the bounds-checked
    # loop with 64-bit addressing; integer-valued entries make the result
    # exact, so it must equal the oracle and the compact layout bit for bit
    M, N, K = 300, 130, 200
    big = (1 << 23) + 64
    d = workloads.random_operands(M, N, K, ta, tb, seed=23, int_range=4)
    compact = run_store(d, ta, tb, M, N, K, out_dtype=torch.float32)
    A = _spread_rows(d["A"], big)
    B = _spread_rows(d["B"], big)
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev())
    tgemm.run(ta, tb, M, N, K, A, big, B, big, C, N, tgemm.EPI_STORE_F32)
    torch.cuda.synchronize()
    del A, B
    ref = oracle_gemm_from(d, ta, tb, M, N, K)
    assert np.array_equal(C.cpu().numpy().astype(np.float64), ref)
    assert torch.equal(C, compact)


def test_identity_gives_op_b():
    K = N = 136
    eye = torch.eye(K, dtype=torch.bfloat16)
    d = workloads.random_operands(K, N, K, "N", "T", seed=5)
    d = dict(d, A=eye, lda=K)
    C = run_store(d, "N", "T", K, N, K)
    assert torch.equal(C.cpu(), d["opB"])


def test_nt_down_projection_full_size():
    """768x5120x13824 NT: X [384,2,13824] flattened by view, W [5120,13824]
    read in place; sampled rows against the oracle."""
    w = workloads.nt_mlp()
    X = w["X"].to(dev())
    W = w["W"].to(dev())
    # a small split-K product through the same kernel first, so that the
    # runtime's per-kernel scratch memory is not counted below
    d = workloads.random_operands(256, 512, 8192, "N", "T", seed=5)
    run_store(d, "N", "T", 256, 512, 8192)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    Y = tgemm.matmul(X, W.t())              # a (1, 13824)-strided view: no copy
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert Y.shape == (384, 2, 5120)
    # torch allocates the output alone (7.9 MB); a transposed copy of W
    # would be 141.6 MB more
    assert torch.cuda.max_memory_allocated() - base < 16 * 2 ** 20
    # new device memory: the output and the split-K partial products the
    # library allocates stream-ordered (4 x 15.7 MB, which the memory pool
    # may round up)
    assert free0 - free1 < 128 * 2 ** 20
    rows = sample_rows(768, 48, seed=2)
    Xb = workloads.bf16_bits(w["X"]).reshape(-1)
    Wb = workloads.bf16_bits(w["W"]).reshape(-1)
    ref = oracle.gemm("N", "T", 768, 5120, 13824, Xb, 13824, Wb, 13824, rows=rows)
    got = bf16_to_f64(Y.view(768, 5120)[torch.as_tensor(rows, device=dev())])
    assert scaled_err(got, ref) <= GEMM_BF16_TOL
    assert rms_rel_err(got, ref) <= GEMM_REL_TOL


@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_layout_sweep_4096(ta, tb):
    M = N = K = 4096
    w = workloads.layout_sweep()
    sa, lda = workloads.store_operand(w["opA"], ta)
    sb, ldb = workloads.store_operand(w["opB"], tb)
    d = {"A": sa, "lda": lda, "B": sb, "ldb": ldb}
    C = run_store(d, ta, tb, M, N, K)
    rows = sample_rows(M, 40, seed=3, tile=256)
    ref = oracle.gemm(ta, tb, M, N, K, bits(sa).reshape(-1), lda, bits(sb).reshape(-1), ldb,
                      rows=rows)
    got = bf16_to_f64(C[torch.as_tensor(rows, device=dev())])
    assert scaled_err(got, ref) <= GEMM_BF16_TOL
    # outputs have RMS ~0.016, far below the 1 of the bar above: bound them
    # relatively too
    assert rms_rel_err(got, ref) <= GEMM_REL_TOL
    # every layout must give the NT bits
    if (ta, tb) != ("N", "T"):
        sa2, lda2 = workloads.store_operand(w["opA"], "N")
        sb2, ldb2 = workloads.store_operand(w["opB"], "T")
        C2 = run_store({"A": sa2, "lda": lda2, "B": sb2, "ldb": ldb2}, "N", "T", M, N, K)
        assert torch.equal(C, C2)


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_k1_store_is_exact_outer_product(out):
    M, N = 333, 77
    for ta, tb in LAYOUTS:
        d = workloads.random_operands(M, N, 1, ta, tb, seed=21, pad=2)
        dt = torch.bfloat16 if out == "bf16" else torch.float32
        C = run_store(d, ta, tb, M, N, 1, out_dtype=dt)
        ref = oracle_gemm_from(d, ta, tb, M, N, 1)      # exact products
        if out == "bf16":
            assert np.array_equal(bits(C), oracle.f64_to_bf16_bits(ref))
        else:
            assert np.array_equal(C.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("cfg", [1, 2, 3])
@pytest.mark.parametrize("split", [2, 3, 4])
@pytest.mark.parametrize("M,N,K", [(256, 512, 4096), (300, 260, 1000), (512, 256, 2112)])
def test_split_k(M, N, K, split, cfg):
    """K cut into chunks, partial tiles added in fixed chunk order: matches
    the oracle, and two runs give the same bits."""
    d = workloads.random_operands(M, N, K, "N", "T", seed=split * 31 + K)
    prev = tgemm.set_split_k(split)
    try:
        a = run_store(d, "N", "T", M, N, K, out_dtype=torch.float32, cfg=cfg)
        b = run_store(d, "N", "T", M, N, K, out_dtype=torch.float32, cfg=cfg)
        c = run_store(d, "N", "T", M, N, K, cfg=cfg, ldc=N + 3)
    finally:
        tgemm.set_split_k(prev)
    assert torch.isnan(c[:, N:].float()).all()          # nothing written past N
    c = c[:, :N]
    assert torch.equal(a, b)
    ref = oracle_gemm_from(d, "N", "T", M, N, K)
    assert scaled_err(a.cpu().numpy(), ref) <= 1e-4
    assert scaled_err(bf16_to_f64(c), ref) <= GEMM_BF16_TOL
    # the bf16 output is the fp32 sum rounded once (to nearest even)
    assert np.array_equal(bits(c), oracle.f64_to_bf16_bits(a.cpu().numpy().astype(np.float64)))


def test_streams_do_not_share_workspace():
    """Split-K calls of different sizes in flight on two streams at once
    (each stream has its own cached workspace) give the bits of the same
    calls made one after another."""
    shapes = [(256, 512, 8192), (512, 256, 6144)]
    ds = [workloads.random_operands(M, N, K, "N", "T", seed=40 + i) for i, (M, N, K) in
          enumerate(shapes)]
    prev = tgemm.set_split_k(4)
    try:
        serial = [run_store(d, "N", "T", M, N, K, out_dtype=torch.float32, cfg=1)
                  for d, (M, N, K) in zip(ds, shapes)]
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        outs = []
        prev_cfg = tgemm.set_tile_config(1)
        try:
            ops = [(d["A"].to(dev()), d["B"].to(dev()), d) for d in ds]
            torch.cuda.synchronize()
            for rep in range(3):
                for (A, B, d), (M, N, K), st in zip(ops, shapes, streams):
                    C = torch.empty(M, N, dtype=torch.float32, device=dev())
                    with torch.cuda.stream(st):
                        tgemm.run("N", "T", M, N, K, A, d["lda"], B, d["ldb"], C, N,
                                  tgemm.EPI_STORE_F32, stream=st.cuda_stream)
                    outs.append(C)
            torch.cuda.synchronize()
        finally:
            tgemm.set_tile_config(prev_cfg)
    finally:
        tgemm.set_split_k(prev)
    for i, C in enumerate(outs):
        assert torch.equal(C, serial[i % 2])


@pytest.mark.parametrize("cfg", [1, 2, 3])
@pytest.mark.parametrize("M,N,K", [(384, 200, 512), (200, 384, 512), (320, 320, 448), (520, 264, 192)])
def test_ragged_k64_layouts_bitwise(M, N, K, cfg):
    """Ragged shapes with K a multiple of 64 (interior tiles on the
    global->LDS paths, edge tiles on the register path): every layout must
    give the bits of TN (both operands MN-contiguous) and NT must match the
    oracle."""
    outs = {}
    for ta, tb in LAYOUTS:
        d = workloads.random_operands(M, N, K, ta, tb, seed=M + N + K)
        outs[ta + tb] = run_store(d, ta, tb, M, N, K, out_dtype=torch.float32, cfg=cfg)
        if ta + tb == "NT":
            ref = oracle_gemm_from(d, ta, tb, M, N, K)
            assert scaled_err(outs["NT"].cpu().numpy(), ref) <= 1e-4
    for k, v in outs.items():
        assert torch.equal(v, outs["TN"]), k


@pytest.mark.parametrize("cfg", [1, 2, 3])
@pytest.mark.parametrize("split", [2, 3])
@pytest.mark.parametrize("M,N,K", [(256, 512, 4096), (384, 200, 1536)])
def test_split_k_all_layouts_bitwise(M, N, K, split, cfg):
    """K cut into chunks in every layout: each chunk starts at a nonzero k
    on the register path's interior loads (M- or N-contiguous operands) and
    on the direct copies (NT).  Every layout gives the NT bits, NT matches
    the oracle, and the bf16 output is the fp32 sum rounded once."""
    outs, outs16 = {}, {}
    prev = tgemm.set_split_k(split)
    try:
        for ta, tb in LAYOUTS:
            d = workloads.random_operands(M, N, K, ta, tb, seed=7 * split + K)
            outs[ta + tb] = run_store(d, ta, tb, M, N, K, out_dtype=torch.float32, cfg=cfg)
            outs16[ta + tb] = run_store(d, ta, tb, M, N, K, cfg=cfg)
            if ta + tb == "NT":
                ref = oracle_gemm_from(d, ta, tb, M, N, K)
    finally:
        tgemm.set_split_k(prev)
    assert scaled_err(outs["NT"].cpu().numpy(), ref) <= 1e-4
    for k in outs:
        assert torch.equal(outs[k], outs["NT"]), k
        assert torch.equal(outs16[k], outs16["NT"]), k
    assert np.array_equal(bits(outs16["NT"]),
                          oracle.f64_to_bf16_bits(outs["NT"].cpu().numpy().astype(np.float64)))
