"""tgemm_run_noalloc (every scratch buffer in the library's fixed per-device
array) against tgemm_run, through the C ABI: the same kernels, so the same
bits.  Each case runs two calls in a row, the second with a smaller input,
so the second reads a scratch array that still holds the first call's
values."""

import numpy as np
import pytest
import torch

import workloads
from layout_aware_gemm_amd import tgemm
from parity_util import dev

pytestmark = pytest.mark.gpu


def both(ta, tb, M, N, K, d, epi, out_dtype=torch.bfloat16, labels=None, grad=False,
         stream=None):
    """(tgemm_run result, tgemm_run_noalloc result) on the same inputs."""
    A, B = d["A"].to(dev()), d["B"].to(dev())
    outs = []
    for fn in (tgemm.run, tgemm.run_noalloc):
        if epi == tgemm.EPI_CE:
            loss = torch.full((M,), float("nan"), dtype=torch.float32, device=dev())
            g = (torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
                 if grad else None)
            fn(ta, tb, M, N, K, A, d["lda"], B, d["ldb"], None, N, epi, labels=labels,
               out_loss=loss, out_grad=g, stream=stream)
            outs.append((loss, g))
        else:
            C = torch.full((M, N), float("nan"), dtype=out_dtype, device=dev())
            fn(ta, tb, M, N, K, A, d["lda"], B, d["ldb"], C, N, epi, stream=stream)
            outs.append(C)
    torch.cuda.synchronize()
    return outs


def test_scratch_size():
    assert tgemm.noalloc_scratch_bytes() == 64 * 2 ** 20


def test_split_k_full_size_then_smaller():
    """The 768x5120x13824 NT product (K split in 4: 60 MiB of fp32 partials
    in the scratch array), then a smaller split product (512x256x4096)."""
    print("noalloc: split-K 768x5120x13824 NT", flush=True)
    w = workloads.nt_mlp()
    d = {"A": w["X"].reshape(768, 13824), "lda": 13824, "B": w["W"], "ldb": 13824}
    ref, got = both("N", "T", 768, 5120, 13824, d, tgemm.EPI_STORE_BF16)
    assert torch.equal(ref, got)
    print("noalloc: split-K 512x256x4096 NT", flush=True)
    d = workloads.random_operands(512, 256, 4096, "N", "T", seed=5)
    ref, got = both("N", "T", 512, 256, 4096, d, tgemm.EPI_STORE_F32, out_dtype=torch.float32)
    assert torch.equal(ref, got)
    assert not torch.isnan(got).any()


@pytest.mark.parametrize("layout", [("N", "T"), ("T", "N")])
def test_cross_entropy_then_smaller(layout):
    """CE with gradient: block partials, label logits and lse in scratch."""
    ta, tb = layout
    for M, N, K in ((1024, 8000, 512), (300, 1000, 64)):
        print(f"noalloc: CE {ta}{tb} {M}x{N}x{K}", flush=True)
        d = workloads.random_operands(M, N, K, ta, tb, seed=M + K)
        labels = torch.randint(0, N, (M,), generator=torch.Generator().manual_seed(N),
                               dtype=torch.int32).to(dev())
        (l0, g0), (l1, g1) = both(ta, tb, M, N, K, d, tgemm.EPI_CE, labels=labels, grad=True)
        assert torch.equal(l0, l1) and torch.equal(g0, g1)
        (l2, _), (l3, _) = both(ta, tb, M, N, K, d, tgemm.EPI_CE, labels=labels)
        assert torch.equal(l2, l3) and torch.equal(l0, l3)


def test_gemv_then_smaller():
    """Matrix-vector products (K-chunk partials in scratch)."""
    for N, K in ((5120, 13824), (300, 1000)):
        print(f"noalloc: gemv 1x{N}x{K}", flush=True)
        d = workloads.random_operands(1, N, K, "N", "T", seed=N)
        ref, got = both("N", "T", 1, N, K, d, tgemm.EPI_STORE_F32, out_dtype=torch.float32)
        assert torch.equal(ref, got)


def test_no_device_memory_is_allocated():
    """On a stream the library has never seen, calls whose scratch needs
    grow (where tgemm_run would allocate a workspace and then grow it) leave
    the device's free memory unchanged.  The stream gets one call first: the
    runtime sets up a new stream's own resources at its first launch."""
    s = torch.cuda.Stream()
    prev = tgemm.set_split_k(4)
    try:
        ops = []
        for M, N, K in ((64, 64, 512), (512, 256, 4096), (768, 1024, 8192)):
            d = workloads.random_operands(M, N, K, "N", "T", seed=M)
            ops.append((M, N, K, d["A"].to(dev()), d["lda"], d["B"].to(dev()), d["ldb"],
                        torch.empty(M, N, dtype=torch.float32, device=dev())))
        torch.cuda.synchronize()

        def call(o):
            M, N, K, A, lda, B, ldb, C = o
            tgemm.run_noalloc("N", "T", M, N, K, A, lda, B, ldb, C, N, tgemm.EPI_STORE_F32,
                              stream=s)

        call(ops[0])
        s.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        for o in ops[1:] + ops[1:]:
            call(o)
        s.synchronize()
        free1 = torch.cuda.mem_get_info()[0]
    finally:
        tgemm.set_split_k(prev)
    assert free1 == free0


def test_too_large_is_rejected_before_any_launch():
    """A split product whose partials exceed the scratch array returns
    TGEMM_ERR_WORKSPACE_LIMIT and writes nothing."""
    M, N, K = 640, 640, 4096
    d = workloads.random_operands(M, N, K, "N", "T", seed=7)
    A, B = d["A"].to(dev()), d["B"].to(dev())
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev())
    prev = tgemm.set_split_k(64)          # 64 x 640 x 640 x 4 B = 100 MiB of partials
    try:
        st = tgemm.run_noalloc("N", "T", M, N, K, A, d["lda"], B, d["ldb"], C, N,
                               tgemm.EPI_STORE_F32, check=False)
    finally:
        tgemm.set_split_k(prev)
    torch.cuda.synchronize()
    assert st == tgemm.TGEMM_ERR_WORKSPACE_LIMIT
    assert torch.isnan(C).all()
    assert "WORKSPACE_LIMIT" in tgemm.status_string(st)
