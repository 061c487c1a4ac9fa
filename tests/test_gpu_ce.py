"""GPU parity of the cross-entropy epilogue against the oracle (C-ABI calls)."""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from layout_aware_gemm_amd import tgemm
from parity_util import (GEMM_BF16_TOL, GEMM_REL_TOL, LOSS_REL_TOL, backward_bound_ratio,
                         bf16_to_f64, bits, dev, grad_check, rel_err, rms_rel_err, sample_rows,
                         scaled_err)

pytestmark = pytest.mark.gpu


def run_ce(A, lda, B, ldb, labels, M, N, K, ta="N", tb="T", grad=False, cfg=0, ldg=None):
    loss = torch.full((M,), float("nan"), dtype=torch.float32, device=dev())
    ldg = N if ldg is None else ldg
    g = torch.full((M, ldg), float("nan"), dtype=torch.bfloat16, device=dev()) if grad else None
    prev = tgemm.set_tile_config(cfg)
    try:
        tgemm.run(ta, tb, M, N, K, A, lda, B, ldb, None, ldg, tgemm.EPI_CE, labels=labels,
                  out_loss=loss, out_grad=g)
    finally:
        tgemm.set_tile_config(prev)
    torch.cuda.synchronize()
    return loss, g


def oracle_ce(d, ta, tb, M, N, K, labels, rows=None):
    y = oracle.gemm(ta, tb, M, N, K, bits(d["A"]).reshape(-1), d["lda"],
                    bits(d["B"]).reshape(-1), d["ldb"], rows=rows)
    lab = labels.numpy() if rows is None else labels.numpy()[rows]
    return oracle.cross_entropy(y, lab)


@pytest.mark.parametrize("cfg", [1, 2])
def test_tiny_ce_config(cfg):
    """A bf16[64,128], W bf16[256,128]; C as fp32, loss and grad."""
    w = workloads.tiny_ce()
    A, W, lab = w["A"].to(dev()), w["W"].to(dev()), w["labels"].to(dev())
    d = {"A": w["A"], "lda": 128, "B": w["W"], "ldb": 128}
    C = torch.empty(64, 256, dtype=torch.float32, device=dev())
    tgemm.run("N", "T", 64, 256, 128, A, 128, W, 128, C, 256, tgemm.EPI_STORE_F32)
    loss, g = run_ce(A, 128, W, 128, lab, 64, 256, 128, grad=True, cfg=cfg)
    ref_loss, ref_grad, _ = oracle_ce(d, "N", "T", 64, 256, 128, w["labels"])
    ref_c = oracle.gemm("N", "T", 64, 256, 128, bits(w["A"]).reshape(-1), 128,
                        bits(w["W"]).reshape(-1), 128)
    assert scaled_err(C.cpu().numpy(), ref_c) <= 1e-5        # fp32 output
    assert rel_err(loss.cpu().numpy(), ref_loss) <= LOSS_REL_TOL
    assert scaled_err(bf16_to_f64(g), ref_grad) <= GEMM_BF16_TOL
    assert grad_check(bf16_to_f64(g), ref_grad, w["labels"].numpy()) <= 1.0
    # grad rows sum to ~0 (two bf16 roundings per element: store, then rescale)
    assert np.abs(bf16_to_f64(g).sum(axis=1)).max() <= 2.0 ** -7 + 1e-4


LAYOUTS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]


@pytest.mark.parametrize("cfg", [1, 2])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (5, 3, 7), (70, 300, 96), (257, 520, 130),
                                   (300, 1000, 64), (129, 64, 1), (512, 768, 256)])
def test_ce_ragged(M, N, K, ta, tb, cfg):
    d = workloads.random_operands(M, N, K, ta, tb, seed=M + N + K, std=1.0, pad=1)
    g = torch.Generator().manual_seed(M * N)
    labels = torch.randint(0, N, (M,), generator=g, dtype=torch.int32)
    loss, gr = run_ce(d["A"].to(dev()), d["lda"], d["B"].to(dev()), d["ldb"], labels.to(dev()),
                      M, N, K, ta, tb, grad=True, cfg=cfg, ldg=N + 3)
    ref_loss, ref_grad, _ = oracle_ce(d, ta, tb, M, N, K, labels)
    l = loss.cpu().numpy()
    if N == 1:
        assert np.all(np.abs(l) <= 1e-6)
    else:
        assert rel_err(l, ref_loss) <= LOSS_REL_TOL
    assert scaled_err(bf16_to_f64(gr[:, :N]), ref_grad) <= GEMM_BF16_TOL
    assert grad_check(bf16_to_f64(gr[:, :N]), ref_grad, labels.numpy()) <= 1.0
    assert torch.isnan(gr[:, N:].float()).all()


@pytest.mark.parametrize("ta,tb", LAYOUTS)
@pytest.mark.parametrize("M,N", [(300, 5000), (7, 3), (64, 32000)])
def test_ce_k1_pointwise(M, N, ta, tb):
    """K = 1 cross-entropy runs on the pointwise path (no matrix cores): the
    logits are the exact products a[m] * b[n]; out-of-range labels give a
    NaN loss and a plain-softmax gradient row."""
    d = workloads.random_operands(M, N, 1, ta, tb, seed=M + N, std=3.0, pad=2)
    g = torch.Generator().manual_seed(N)
    labels = torch.randint(0, N, (M,), generator=g, dtype=torch.int32)
    labels[M // 2] = N          # out of range
    loss, gr = run_ce(d["A"].to(dev()), d["lda"], d["B"].to(dev()), d["ldb"], labels.to(dev()),
                      M, N, 1, ta, tb, grad=True, ldg=N + 3)
    ref_loss, ref_grad, _ = oracle_ce(d, ta, tb, M, N, 1, labels)
    l = loss.cpu().numpy()
    bad = np.arange(M) == M // 2
    assert np.isnan(l[bad]).all() and np.isfinite(l[~bad]).all()
    assert rel_err(l[~bad], ref_loss[~bad]) <= LOSS_REL_TOL
    gg = bf16_to_f64(gr[:, :N])
    assert scaled_err(gg, ref_grad) <= GEMM_BF16_TOL
    assert grad_check(gg, ref_grad, labels.numpy()) <= 1.0
    assert torch.isnan(gr[:, N:].float()).all()
    # loss only gives the same losses
    l2, _ = run_ce(d["A"].to(dev()), d["lda"], d["B"].to(dev()), d["ldb"], labels.to(dev()),
                   M, N, 1, ta, tb)
    assert np.array_equal(l2.cpu().numpy(), l, equal_nan=True)


def test_zero_logits_give_ln_n():
    M, N, K = 64, 32000, 64
    A = torch.zeros(M, K, dtype=torch.bfloat16, device=dev())
    W = torch.randn(N, K, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).to(dev())
    labels = torch.randint(0, N, (M,), generator=torch.Generator().manual_seed(2),
                           dtype=torch.int32)
    loss, g = run_ce(A, K, W, K, labels.to(dev()), M, N, K, grad=True)
    assert np.abs(loss.cpu().numpy() - math.log(N)).max() <= 1e-3 * math.log(N)
    gg = bf16_to_f64(g)
    onehot = np.zeros((M, N))
    onehot[np.arange(M), labels.numpy()] = 1
    assert scaled_err(gg, 1.0 / N - onehot) <= GEMM_BF16_TOL
    assert grad_check(gg, 1.0 / N - onehot, labels.numpy()) <= 1.0


def test_out_of_range_labels_give_nan():
    M, N, K = 8, 300, 32
    d = workloads.random_operands(M, N, K, "N", "T", seed=4)
    labels = torch.tensor([0, 299, 300, -1, 5, 1 << 30, 7, 150], dtype=torch.int32)
    loss, g = run_ce(d["A"].to(dev()), K, d["B"].to(dev()), K, labels.to(dev()), M, N, K,
                     grad=True)
    l = loss.cpu().numpy()
    bad = np.array([False, False, True, True, False, True, False, False])
    assert np.all(np.isnan(l[bad])) and np.all(np.isfinite(l[~bad]))
    ref_loss, ref_grad, _ = oracle_ce(d, "N", "T", M, N, K, labels)
    assert rel_err(l[~bad], ref_loss[~bad]) <= LOSS_REL_TOL
    assert scaled_err(bf16_to_f64(g), ref_grad) <= GEMM_BF16_TOL
    assert grad_check(bf16_to_f64(g), ref_grad, labels.numpy()) <= 1.0


@pytest.mark.parametrize("cfg", [1, 2])
def test_nan_logit_propagates_to_its_row(cfg):
    """A NaN in row i of A makes every logit of row i NaN: that row's loss
    and gradient row are NaN (the oracle's fp64 result is NaN too), and the
    other rows still match the oracle."""
    M, N, K = 70, 600, 64
    d = workloads.random_operands(M, N, K, "N", "T", seed=12)
    A = d["A"].clone()
    A[5, 3] = float("nan")
    labels = torch.randint(0, N, (M,), generator=torch.Generator().manual_seed(8),
                           dtype=torch.int32)
    loss, g = run_ce(A.to(dev()), K, d["B"].to(dev()), K, labels.to(dev()), M, N, K, grad=True,
                     cfg=cfg)
    l = loss.cpu().numpy()
    ref_loss, ref_grad, _ = oracle_ce({"A": A, "lda": K, "B": d["B"], "ldb": K}, "N", "T", M, N,
                                      K, labels)
    assert np.isnan(ref_loss[5]) and np.isnan(l[5])
    gg = bf16_to_f64(g)
    assert np.all(np.isnan(gg[5]))
    ok = np.arange(M) != 5
    assert np.all(np.isfinite(l[ok]))
    assert rel_err(l[ok], ref_loss[ok]) <= LOSS_REL_TOL
    assert scaled_err(gg[ok], ref_grad[ok]) <= GEMM_BF16_TOL
    assert grad_check(gg[ok], ref_grad[ok], labels.numpy()[ok]) <= 1.0


def test_ce_deterministic_and_grad_mode_same_loss():
    M, N, K = 512, 3000, 256
    d = workloads.random_operands(M, N, K, "N", "T", seed=9)
    labels = torch.randint(0, N, (M,), generator=torch.Generator().manual_seed(3),
                           dtype=torch.int32).to(dev())
    A, B = d["A"].to(dev()), d["B"].to(dev())
    l0, _ = run_ce(A, K, B, K, labels, M, N, K)
    for _ in range(5):
        l1, _ = run_ce(A, K, B, K, labels, M, N, K)
        assert torch.equal(l0, l1)
    l2, _ = run_ce(A, K, B, K, labels, M, N, K, grad=True)
    assert torch.equal(l0, l2)


def test_ce_vocab_full_size():
    """H bf16[4096,4096], W bf16[32000,4096], labels in [0,32000): loss-only
    and loss+grad, sampled rows against the oracle."""
    w = workloads.ce_vocab()
    H, W, lab = w["H"].to(dev()), w["W"].to(dev()), w["labels"].to(dev())
    M, N, K = 4096, 32000, 4096
    loss = tgemm.cross_entropy(H, W.t(), lab)
    loss2, g = tgemm.cross_entropy(H, W.t(), lab, grad=True)
    torch.cuda.synchronize()
    assert torch.equal(loss, loss2)
    rows = sample_rows(M, 24, seed=4, tile=256)
    d = {"A": w["H"], "lda": K, "B": w["W"], "ldb": K}
    ref_loss, ref_grad, _ = oracle_ce(d, "N", "T", M, N, K, w["labels"], rows=rows)
    r = torch.as_tensor(rows, device=dev())
    assert rel_err(loss[r].cpu().numpy(), ref_loss) <= LOSS_REL_TOL
    assert scaled_err(bf16_to_f64(g[r]), ref_grad) <= GEMM_BF16_TOL
    assert grad_check(bf16_to_f64(g[r]), ref_grad, w["labels"].numpy()[rows]) <= 1.0
    # every row of the gradient sums to ~0 and every loss is positive
    sums = g.float().sum(dim=1)
    assert sums.abs().max().item() <= 2.0 ** -7 + 1e-3
    assert (loss > 0).all().item()


def oracle_grad_bf16(y, labels):
    """The oracle's softmax - onehot, rounded once to bf16 (as fp64 values)."""
    _, grad, _ = oracle.cross_entropy(y, labels)
    return oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(grad))


def test_ce_backward_gemms_full_size():
    """The two GEMMs that consume the gradient G = softmax - onehot of the
    fused CE, each reading its operands as stored: dH = G . W is an NN call
    (W stored [32000, 4096] is op(B) as is), dW = G^T . H a TN call (G read
    transposed in place).  dH's sampled rows against the oracle's own
    gradient (its bf16 rounding of softmax - onehot) times W; the GPU
    gradient carries one more rounding, which the bound accounts for."""
    w = workloads.ce_vocab()
    H, W, lab = w["H"].to(dev()), w["W"].to(dev()), w["labels"].to(dev())
    M, N, K = 4096, 32000, 4096
    _, G = tgemm.cross_entropy(H, W.t(), lab, grad=True)
    dH = tgemm.matmul(G, W)            # [4096, 32000] . [32000, 4096]
    dW = tgemm.matmul(G.t(), H)        # [32000, 4096] . [4096, 4096]
    torch.cuda.synchronize()
    assert tgemm.layout_of(G)[0] == "N" and tgemm.layout_of(W)[0] == "N"
    assert tgemm.layout_of(G.t())[0] == "T" and tgemm.layout_of(H)[0] == "N"
    rows = sample_rows(M, 12, seed=6, tile=512)
    d = {"A": w["H"], "lda": K, "B": w["W"], "ldb": K}
    y = oracle.gemm("N", "T", M, N, K, bits(d["A"]).reshape(-1), K, bits(d["B"]).reshape(-1), K,
                    rows=rows)
    g_ref = oracle_grad_bf16(y, w["labels"].numpy()[rows])
    Wf = oracle.bf16_bits_to_f64(workloads.bf16_bits(w["W"]))
    ref = g_ref @ Wf
    got = bf16_to_f64(dH[torch.as_tensor(rows, device=dev())])
    assert scaled_err(got, ref) <= GEMM_BF16_TOL
    assert backward_bound_ratio(got, g_ref, Wf, ref) <= 1.0
    # dW: every element needs a whole column of G (all 4096 rows' lse), so
    # the oracle check runs at a reduced size (test_ce_backward_oracle);
    # here: the deferred route gives the same bits (test below) and dW is
    # finite with the sum of its rows equal to the column sums of G^T H
    assert torch.isfinite(dW.float()).all()


@pytest.mark.parametrize("M,V,K", [(512, 4000, 512), (300, 1000, 130)])
def test_ce_backward_oracle(M, V, K):
    """dH = G . W and dW = G^T . H against the oracle's own gradient, for the
    rescale-pass route (tgemm_run on the finished gradient) and the
    deferred route (tgemm_run_ce_grad finishing it on load), which must
    agree bit for bit."""
    g = torch.Generator().manual_seed(M + V)
    Hh = torch.randn(M, K, generator=g).to(torch.bfloat16)
    Wv = (torch.randn(V, K, generator=g) * 0.2).to(torch.bfloat16)
    labels = torch.randint(0, V, (M,), generator=g, dtype=torch.int32)
    labels[M // 3] = V + 5                     # out of range: no one-hot term
    Hd, Wd, ld = Hh.to(dev()), Wv.to(dev()), labels.to(dev())
    loss, G = tgemm.cross_entropy(Hd, Wd.t(), ld, grad=True)
    loss2, E, S = tgemm.cross_entropy_deferred(Hd, Wd.t(), ld)
    dH = tgemm.matmul(G, Wd)
    dW = tgemm.matmul(G.t(), Hd)
    dH2 = tgemm.ce_grad_matmul(E, S, ld, Wd)
    dW2 = tgemm.ce_grad_matmul(E.t(), S, ld, Hd)
    torch.cuda.synchronize()
    # (the out-of-range row's loss is NaN on both routes)
    assert torch.allclose(loss, loss2, rtol=0, atol=0, equal_nan=True)
    assert torch.isnan(loss[M // 3]).item()
    assert torch.equal(dH, dH2) and torch.equal(dW, dW2)
    y = oracle.gemm("N", "T", M, V, K, workloads.bf16_bits(Hh).reshape(-1), K,
                    workloads.bf16_bits(Wv).reshape(-1), K)
    g_ref = oracle_grad_bf16(y, labels.numpy())
    Hf = oracle.bf16_bits_to_f64(workloads.bf16_bits(Hh))
    Wf = oracle.bf16_bits_to_f64(workloads.bf16_bits(Wv))
    for got, gr, other in ((dH, g_ref, Wf), (dW, g_ref.T, Hf)):
        ref = gr @ other
        gg = bf16_to_f64(got)
        assert scaled_err(gg, ref) <= GEMM_BF16_TOL
        assert backward_bound_ratio(gg, gr, other, ref) <= 1.0


@pytest.mark.parametrize("cfg", [0, 1, 2])
@pytest.mark.parametrize("tb", ["N", "T"])
# (576, 832, 256, 320): odd k-step counts (13 for G . Y, 9 for G^T . Z) on
# the 256x256 interior tiles, where a zero k-step pads the two-set loop,
# and 64 x 64 blocks of which many hold a label column
@pytest.mark.parametrize("M,V,K,X", [(257, 520, 130, 200), (64, 256, 128, 96), (512, 768, 256, 384),
                                     (576, 832, 256, 320)])
def test_ce_grad_on_load_equals_rescale_pass(M, V, K, X, tb, cfg):
    """Every layout and tile configuration of tgemm_run_ce_grad against
    tgemm_run on the finished gradient, bit for bit (bf16 and fp32 out);
    the gradient read as G and as G^T."""
    d = workloads.random_operands(M, V, K, "N", "T", seed=M + V + K, std=1.0)
    g = torch.Generator().manual_seed(X)
    labels = torch.randint(0, V, (M,), generator=g, dtype=torch.int32)
    # two rows whose labels fall outside [0, V): no one-hot term on either
    # route (the losses are NaN, the gradients still defined)
    labels[0] = -1
    labels[M - 1] = V
    labels = labels.to(dev())
    A, B = d["A"].to(dev()), d["B"].to(dev())
    loss, G = tgemm.cross_entropy(A, B.t(), labels, grad=True)
    _, E, S = tgemm.cross_entropy_deferred(A, B.t(), labels)
    other_h = torch.randn(V, X, generator=g).to(torch.bfloat16).to(dev())   # for G . Y
    other_w = torch.randn(M, X, generator=g).to(torch.bfloat16).to(dev())   # for G^T . Z
    if tb == "T":
        other_h = other_h.t().contiguous().t()
        other_w = other_w.t().contiguous().t()
    prev = tgemm.set_tile_config(cfg)
    try:
        for out_dtype in (torch.bfloat16, torch.float32):
            a = tgemm.matmul(G, other_h, out_dtype=out_dtype)
            b = tgemm.ce_grad_matmul(E, S, labels, other_h, out_dtype=out_dtype)
            c = tgemm.matmul(G.t(), other_w, out_dtype=out_dtype)
            e = tgemm.ce_grad_matmul(E.t(), S, labels, other_w, out_dtype=out_dtype)
            torch.cuda.synchronize()
            assert torch.equal(a, b) and torch.equal(c, e)
    finally:
        tgemm.set_tile_config(prev)


def test_ce_deferred_full_size_same_bits():
    """At 4096 x 32000 x 4096: the deferred loss equals the loss of the
    rescale-pass route, and dH, dW finished on load equal dH, dW of the
    finished gradient, bit for bit."""
    w = workloads.ce_vocab()
    H, W, lab = w["H"].to(dev()), w["W"].to(dev()), w["labels"].to(dev())
    loss, G = tgemm.cross_entropy(H, W.t(), lab, grad=True)
    dH = tgemm.matmul(G, W)
    dW = tgemm.matmul(G.t(), H)
    del G
    loss2, E, S = tgemm.cross_entropy_deferred(H, W.t(), lab)
    dH2 = tgemm.ce_grad_matmul(E, S, lab, W)
    dW2 = tgemm.ce_grad_matmul(E.t(), S, lab, H)
    torch.cuda.synchronize()
    assert torch.equal(loss, loss2)
    assert torch.equal(dH, dH2) and torch.equal(dW, dW2)
