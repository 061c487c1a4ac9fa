"""Shared helpers for the GPU parity tests (comparison only, no method math)."""

import numpy as np
import torch

import oracle
import workloads

# Parity bars of this project.
GEMM_BF16_TOL = 1e-2     # max |gpu - ref| / (|ref| + 1) for bf16 matrix outputs
LOSS_REL_TOL = 1e-3      # per-row loss, relative
K1_F32_ABS_TOL = 1e-5    # K=1 fp32 table, absolute
TRIG_ABS_TOL = 2.0 ** -8  # bf16 cos/sin tables, absolute (1 bf16 ulp in [0.5, 1))
# Relative bars scaled to each output's own size.  A bf16 value carries one
# rounding of at most 2^-9 relative; the gradient carries two (the stored
# exp(y - block max), then the rescale), so 2^-7 leaves a factor 2 of margin
# over both, while a wrong value (a uniform or permuted softmax, a scaled
# product) misses it by far.
GRAD_REL_TOL = 2.0 ** -7
GRAD_FLOOR = 2.0 ** -120  # fp32 exponentials of logits ~87 below the row max underflow
GEMM_REL_TOL = 2.0 ** -8  # max |gpu - ref| / (|ref| + rms(ref)/64) for bf16 products


def dev():
    return torch.device("cuda:0")


def bits(t):
    """Any bf16 tensor (GPU or CPU) -> NumPy uint16 bits."""
    return workloads.bf16_bits(t.detach().cpu())


def bf16_to_f64(t):
    return oracle.bf16_bits_to_f64(bits(t))


def scaled_err(gpu, ref):
    """max |gpu - ref| / (|ref| + 1)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if gpu.size == 0:
        return 0.0
    return float(np.max(np.abs(gpu - ref) / (np.abs(ref) + 1.0)))


def rel_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(gpu - ref) / np.abs(ref)))


def oracle_gemm_from(d, ta, tb, M, N, K, rows=None):
    """Oracle C for a workloads.random_operands-style dict (stored operands)."""
    return oracle.gemm(ta, tb, M, N, K, bits(d["A"]).reshape(-1), d["lda"],
                       bits(d["B"]).reshape(-1), d["ldb"], rows=rows)


def sample_rows(M, n, seed, tile=128):
    """Rows spread over every M tile, including the first and last row."""
    rng = np.random.default_rng(seed)
    rows = set([0, M - 1])
    for t0 in range(0, M, tile):
        rows.add(int(rng.integers(t0, min(M, t0 + tile))))
    while len(rows) < min(n, M):
        rows.add(int(rng.integers(0, M)))
    return np.array(sorted(rows))


def grad_check(g_gpu, grad_ref, labels):
    """Worst ratio of error to bound (<= 1 passes) of a softmax-minus-one-hot
    gradient against the oracle's fp64 one.

    Off the label column the probabilities themselves are compared
    relatively: |g_gpu - g_ref| <= GRAD_REL_TOL * p_ref + GRAD_FLOOR, with
    p_ref the oracle softmax.  At the label column g = p - 1, whose value
    carries the roundings of both p and g:
    |g_gpu - g_ref| <= GRAD_REL_TOL * max(p_ref, |g_ref|) + GRAD_FLOOR.
    Rows with a label outside [0, N) have no one-hot term.
    """
    g = np.asarray(g_gpu, dtype=np.float64)
    ref = np.asarray(grad_ref, dtype=np.float64)
    if g.size == 0:
        return 0.0
    M, N = ref.shape
    lab = np.asarray(labels).astype(np.int64).reshape(M)
    onehot = np.zeros((M, N))
    hit = np.flatnonzero((lab >= 0) & (lab < N))
    onehot[hit, lab[hit]] = 1.0
    p_ref = ref + onehot
    bound = GRAD_REL_TOL * np.maximum(p_ref, np.abs(ref) * onehot) + GRAD_FLOOR
    return float(np.max(np.abs(g - ref) / bound))


def rms_rel_err(gpu, ref):
    """max |gpu - ref| / (|ref| + rms(ref)/64): relative for every output not
    far below the output's typical size, with a floor at 1/64 of its RMS
    (fp32 accumulation error is orders of magnitude smaller)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if gpu.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(gpu - ref) / (np.abs(ref) + rms / 64.0)))


def backward_bound_ratio(got, g_ref, other, ref):
    """Worst ratio of |got - ref| to the bound the arithmetic allows, for a
    product ref = g_ref @ other of a gradient with the oracle's (one bf16
    rounding of softmax - onehot): the GPU gradient differs from it by at
    most two roundings, 2^-8 relative per element, so the product by at most
    2^-8 (|g_ref| @ |other|); the bf16 output adds 2^-9 |ref|.  The bound is
    taken at twice that."""
    bound = 2.0 ** -7 * (np.abs(g_ref) @ np.abs(other)) + 2.0 ** -8 * np.abs(ref) + 1e-30
    return float(np.max(np.abs(got - ref) / bound))


# ---- fp8 products (tgemm_run_fp8) -------------------------------------------
# The packed route multiplies on the fp8 matrix cores, which add the products
# of each group of 8 consecutive k at the magnitude of the group's largest
# product, truncating the others' bits below about 2^-12 of it (measured on
# MI355X with structured inputs).  Each group thus adds at most
# 2^-9 * max |qa qb| over the group beyond the fp32 summation bound.
FP8_RMS_F32 = 2.0 ** -10   # rms(gpu - ref) / rms(ref), fp32 outputs
FP8_RMS_BF16 = 2.0 ** -8   # the same with one bf16 rounding


def fp8_quantized(d, scales, rows=None):
    """|qa| (rows of op(A), optionally a subset) and |qb| in fp64; NaN -> 0."""
    sa, sb, _ = scales
    qa = np.abs(oracle.quantize(np.nan_to_num(d["opA"].float().numpy()), sa))
    qb = np.abs(oracle.quantize(np.nan_to_num(d["opB"].float().numpy()), sb))
    if rows is not None:
        qa = qa[np.asarray(rows)]
    return qa, qb


def fp8_group_loss_bound(qa, qb):
    """sum over groups of 8 consecutive k of 2^-9 * max |qa qb| in the group,
    per output element ([rows, N]); qa [R, K] and qb [K, N] nonnegative."""
    R, K = qa.shape
    Kg = -(-K // 8) * 8
    qa = np.pad(qa, ((0, 0), (0, Kg - K)))
    qb = np.pad(qb, ((0, Kg - K), (0, 0)))
    out = np.empty((R, qb.shape[1]))
    for r in range(R):
        p = qa[r][:, None] * qb
        out[r] = p.reshape(Kg // 8, 8, -1).max(axis=1).sum(axis=0)
    return out * 2.0 ** -9


def fp8_error_bound(d, scales, K, ref, rows=None, packed=False):
    """Per-element bound on |C - ref| for an fp8 product with output scale
    scales[2]: the fp32 summation bound, plus the group loss when packed."""
    qa, qb = fp8_quantized(d, scales, rows)
    so = abs(scales[2])
    bound = K * 2.0 ** -24 * (qa @ qb) * so * 1.01 + np.abs(ref) * 2.0 ** -23 + 1e-30
    if packed:
        bound = bound + fp8_group_loss_bound(qa, qb) * so
    return bound


def within_bound(C, ref, bound):
    return bool(np.all(np.abs(np.asarray(C, dtype=np.float64) - ref) <= bound))


def rms_ratio(gpu, ref):
    """rms(gpu - ref) / rms(ref)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.sqrt(np.mean((gpu - ref) ** 2)) / np.sqrt(np.mean(ref * ref)))
