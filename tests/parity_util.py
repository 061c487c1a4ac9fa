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
