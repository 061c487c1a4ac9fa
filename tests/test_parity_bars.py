"""The relative parity bars reject plausible wrong answers (CPU only).

Negative controls for the checks the GPU tests apply at the workloads'
real scales: at the tiny CE (64x256x128) and the fused CE (4096x32000x4096)
the softmax entries are at most about 1e-2, and the 4096^3 layout-sweep
outputs have RMS about 0.016, so the absolute-style bar
max |gpu - ref| / (|ref| + 1) <= 1e-2 alone would pass a gradient that
ignores the logits or an output scaled by 0.85.  The relative bars must
fail each such answer and pass the oracle's own values after the roundings
a correct bf16 result carries.
"""

import numpy as np

import oracle
import workloads
from parity_util import (FP8_RMS_BF16, FP8_RMS_F32, GEMM_BF16_TOL, GEMM_REL_TOL,
                         backward_bound_ratio, fp8_error_bound, grad_check, rms_ratio,
                         rms_rel_err, sample_rows, scaled_err, within_bound)


def onehot_of(labels, N):
    lab = np.asarray(labels).astype(np.int64)
    oh = np.zeros((lab.size, N))
    oh[np.arange(lab.size), lab] = 1.0
    return oh


def wrong_gradients(ref, labels):
    """Wrong answers that keep every row summing to zero."""
    M, N = ref.shape
    oh = onehot_of(labels, N)
    p = ref + oh
    return {
        "uniform": np.full((M, N), 1.0 / N) - oh,                # ignores the logits
        "permuted": np.roll(p, 1, axis=1) - oh,                  # columns shifted by one
        "scaled": 0.85 * p - oh * 0.85,                          # wrong scale
        "sharpened": p ** 1.1 / (p ** 1.1).sum(1, keepdims=True) - oh,  # wrong temperature
    }


def right_gradients(ref, labels):
    """The oracle's gradient after a correct bf16 result's roundings: once,
    and with the two roundings' worst case (each probability off by 2^-8
    relative, in either direction)."""
    N = ref.shape[1]
    oh = onehot_of(labels, N)
    p = ref + oh
    once = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(ref))
    up = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(p * (1 + 2.0 ** -8) - oh))
    down = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(p * (1 - 2.0 ** -8) - oh))
    return {"once": once, "up": up, "down": down}


def check_gradient_bars(y, labels):
    _, ref, _ = oracle.cross_entropy(y, labels)
    for name, g in right_gradients(ref, labels).items():
        assert grad_check(g, ref, labels) <= 1.0, name
    for name, g in wrong_gradients(ref, labels).items():
        # the old absolute-style bar is blind to every one of them ...
        if name in ("uniform", "permuted"):
            assert scaled_err(g, ref) <= GEMM_BF16_TOL, name
        # ... the relative one is not
        assert grad_check(g, ref, labels) > 4.0, name


def test_tiny_ce_gradient_bar_rejects_wrong_gradients():
    w = workloads.tiny_ce()
    y = oracle.gemm("N", "T", 64, 256, 128, workloads.bf16_bits(w["A"]).reshape(-1), 128,
                    workloads.bf16_bits(w["W"]).reshape(-1), 128)
    check_gradient_bars(y, w["labels"].numpy())


def test_fused_ce_gradient_bar_rejects_wrong_gradients():
    w = workloads.ce_vocab()
    rows = sample_rows(4096, 8, seed=4, tile=1024)
    y = oracle.gemm("N", "T", 4096, 32000, 4096, workloads.bf16_bits(w["H"]).reshape(-1), 4096,
                    workloads.bf16_bits(w["W"]).reshape(-1), 4096, rows=rows)
    check_gradient_bars(y, w["labels"].numpy()[rows])


def test_label_column_bar():
    """At the label column g = p - 1: a label entry that forgot the one-hot
    term, or subtracted it twice, fails; a probability near 1 is allowed its
    rounding."""
    y = np.array([[8.0, 0.0, -1.0, 0.5], [0.0, 0.1, 0.2, 0.3]])
    labels = np.array([0, 2])
    _, ref, _ = oracle.cross_entropy(y, labels)
    ok = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(ref))
    assert grad_check(ok, ref, labels) <= 1.0
    bad = ref.copy()
    bad[1, 2] += 1.0                 # the one-hot term missing
    assert grad_check(bad, ref, labels) > 4.0
    bad = ref.copy()
    bad[0, 0] -= 1.0                 # subtracted twice
    assert grad_check(bad, ref, labels) > 4.0


def test_layout_sweep_bar_rejects_scaled_or_shifted_products():
    ls = workloads.layout_sweep()
    sa, lda = workloads.store_operand(ls["opA"], "N")
    sb, ldb = workloads.store_operand(ls["opB"], "T")
    rows = sample_rows(4096, 12, seed=3, tile=1024)
    ref = oracle.gemm("N", "T", 4096, 4096, 4096, workloads.bf16_bits(sa).reshape(-1), lda,
                      workloads.bf16_bits(sb).reshape(-1), ldb, rows=rows)
    rounded = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(ref))
    assert rms_rel_err(rounded, ref) <= GEMM_REL_TOL
    # a value off by one bf16 step and a half still passes; the bar is not tighter
    # than the output format
    assert rms_rel_err(ref * (1 + 2.0 ** -9), ref) <= GEMM_REL_TOL
    # the absolute-style bar sits near its limit for an output scaled by
    # 0.85 (about 0.012 against 0.01 on these rows); the relative bar misses
    # every wrong answer by far
    for wrong in (0.85 * ref, 0.98 * ref, np.roll(ref, 1, axis=1), ref[::-1]):
        assert rms_rel_err(wrong, ref) > 4 * GEMM_REL_TOL


def test_backward_bound_rejects_wrong_products():
    """The bound used for the CE backward GEMMs (2^-7 |G| @ |W| + 2^-8 |ref|)
    passes the product of the gradient after two bf16 roundings and rejects
    a gradient that ignores the logits, a scaled one, and a product with the
    wrong operand order."""
    rng = np.random.default_rng(1)
    M, V, K = 64, 300, 48
    y = rng.normal(size=(M, V)) * 2
    labels = rng.integers(0, V, M)
    W = rng.normal(size=(V, K)) * 0.2
    _, grad, _ = oracle.cross_entropy(y, labels)
    g1 = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(grad))
    ref = g1 @ W
    oh = onehot_of(labels, V)
    p = grad + oh
    g2 = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(
        oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(p * (1 + 2.0 ** -9))) - oh))
    got = oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(g2 @ W))
    assert backward_bound_ratio(got, g1, W, ref) <= 1.0
    uniform = (np.full((M, V), 1.0 / V) - oh) @ W
    assert backward_bound_ratio(uniform, g1, W, ref) > 4.0
    assert backward_bound_ratio(0.9 * ref, g1, W, ref) > 4.0
    assert backward_bound_ratio(np.roll(ref, 1, axis=0), g1, W, ref) > 4.0


def group_truncated_sum(qa, qb, shift):
    """A plausible fp8 matrix-core result: in each group of 8 consecutive k,
    every product truncated toward zero to a multiple of 2^(E - shift), E the
    exponent of the group's largest |product|; exact sums otherwise."""
    R, K = qa.shape
    p = qa[:, :, None] * qb[None, :, :]
    p = p.reshape(R, K // 8, 8, -1)
    mx = np.abs(p).max(axis=2, keepdims=True)
    u = 2.0 ** (np.floor(np.log2(np.where(mx > 0, mx, 1.0))) - shift)
    return (np.trunc(p / u) * u).sum(axis=(1, 2))


def test_fp8_packed_bars_reject_wrong_products():
    """The fp8 packed route's checks (per-element bound with the group loss,
    and the RMS ratio) pass the oracle's product and products truncated as
    the fp8 matrix cores do (at the measured 2^-12 and at twice that), in
    fp32 and after a bf16 rounding, and reject a 0.99x product, one group of
    8 k left out, shifted columns and the e4m3fn cast skipped."""
    rng = np.random.default_rng(4)
    R, K, N = 6, 512, 192
    x = rng.normal(size=(R, K))
    w = rng.normal(size=(K, N)) * 0.02
    sa, sb = 10.0, 1000.0
    so = 1.0 / (sa * sb)
    import torch
    d = {"opA": torch.tensor(x), "opB": torch.tensor(w)}
    qa, qb = oracle.quantize(x, sa), oracle.quantize(w, sb)
    ref = (qa @ qb) * so
    bound = fp8_error_bound(d, (sa, sb, so), K, ref, packed=True)

    def bf16(v):
        return oracle.bf16_bits_to_f64(oracle.f64_to_bf16_bits(v))

    for shift in (12, 11):
        got = group_truncated_sum(qa, qb, shift) * so
        assert within_bound(got, ref, bound) and rms_ratio(got, ref) <= FP8_RMS_F32
        gb = bf16(got)
        assert within_bound(gb, ref, bound + np.abs(ref) * 2.0 ** -8)
        assert rms_ratio(gb, ref) <= FP8_RMS_BF16
    gap = qa.copy()
    gap[:, 64:72] = 0
    wrong = {
        "scaled": 0.99 * ref,
        "group left out": (gap @ qb) * so,
        "shifted columns": np.roll(ref, 1, axis=1),
        "no cast": (x * sa) @ (w * sb) * so,
    }
    for name, v in wrong.items():
        assert not within_bound(v, ref, bound), name
        assert rms_ratio(v, ref) > 4 * FP8_RMS_F32, name
        assert rms_ratio(bf16(v), ref) > 2 * FP8_RMS_BF16, name
