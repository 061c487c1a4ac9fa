"""Graph capture: calls made while their stream is being captured allocate
their workspace in stream order inside the graph.  A captured split-K NT
product and a cross-entropy call with gradient are replayed several times,
with eager work on the same buffers between replays; every replay must give
the bits of the eager calls."""

import pytest
import torch

import workloads
from layout_aware_gemm_amd import tgemm
from parity_util import dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    M, N, K = 256, 512, 8192            # 2 tiles of 256x256: K split into 4 chunks
    d = workloads.random_operands(M, N, K, "N", "T", seed=77)
    A, B = d["A"].to(dev()), d["B"].to(dev())
    C = torch.empty(M, N, dtype=torch.bfloat16, device=dev())
    w = workloads.tiny_ce()
    H, W, lab = w["A"].to(dev()), w["W"].to(dev()), w["labels"].to(dev())
    loss = torch.empty(64, dtype=torch.float32, device=dev())
    grad = torch.empty(64, 256, dtype=torch.bfloat16, device=dev())

    def calls():
        tgemm.run("N", "T", M, N, K, A, d["lda"], B, d["ldb"], C, N, tgemm.EPI_STORE_BF16)
        tgemm.run("N", "T", 64, 256, 128, H, 128, W, 128, None, 256, tgemm.EPI_CE,
                  labels=lab, out_loss=loss, out_grad=grad)

    calls()
    torch.cuda.synchronize()
    C_ref, loss_ref, grad_ref = C.clone(), loss.clone(), grad.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                          # a call on the capture stream before capturing
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work on the outputs between replays
        C.fill_(float("nan"))
        loss.fill_(float("nan"))
        grad.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, C_ref), rep
        assert torch.equal(loss, loss_ref), rep
        assert torch.equal(grad, grad_ref), rep


def test_graph_replays_fp8_cast_once():
    # 520 x 536 x 256 fp8 product: the cast-once route, whose two cast
    # passes write into a workspace allocated inside the graph
    M, N, K = 520, 536, 256
    d = workloads.random_operands(M, N, K, "N", "T", seed=78, std=3.0)
    A, B = d["A"].to(dev()), d["B"].to(dev())
    sc = torch.tensor([4.0, 8.0, 1.0 / 32], dtype=torch.float32, device=dev())
    C = torch.empty(M, N, dtype=torch.bfloat16, device=dev())

    def call():
        tgemm.run_fp8("N", "T", M, N, K, A, d["lda"], B, d["ldb"], C, N, tgemm.EPI_STORE_BF16,
                      sc)

    call()
    torch.cuda.synchronize()
    C_ref = C.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        C.fill_(float("nan"))
        A.add_(0)                         # eager work on the inputs between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, C_ref), rep
