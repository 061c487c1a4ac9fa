"""Oracle row-wise cross-entropy on GEMM logits (test infrastructure only).

What is computed ("Allow reductions in matmul epilogues", the attempted
fusion, whose comment defines the loss, and its edit note on the gradient
kept for the backward pass): for logits y[M, N] and one integer label per
row,

    loss[m] = logsumexp(y[m, :]) - y[m, label[m]]
    grad[m, n] = softmax(y[m, :])[n] - [n == label[m]]

written here from those definitions in fp64 (the logits are never rounded
to bf16 first).  logsumexp is evaluated with the usual shift by the row
maximum so that large logits neither overflow nor lose the small terms.

Readings where the page is garbled or silent:

* Loss.  The page's comment gives lse minus the label logit, while its code
  broadcasts lse across the row before summing (which would give
  N*lse - y[label]).  The comment and the definition of cross-entropy
  agree, so loss = lse - y[label].  For N = 1 both readings coincide.
* One loss per row: no mean over rows, no scaling of the gradient, no ignore
  index, no label smoothing.
* Labels outside [0, N) are not defined by the page.  Here such a row gets a
  NaN loss and its gradient row is the plain softmax (no one-hot term).

The tile-wise combine ("Allow reductions in matmul epilogues", the question
about row-wise reductions when the matmul runs tile by tile, and its answer:
a grid reduction through atomics or semaphores) is written out as
``tile_partials`` + ``merge_partials``: each tile of columns yields a
(max, sum of exp shifted by that max) pair and pairs merge by rescaling both
sums to the larger max.  The merge identity is (-inf, 0).
"""

import numpy as np


def logsumexp_rows(y):
    """log(sum_n exp(y[m, n])) for every row m of a 2-D fp64 array."""
    peak = y.max(axis=1)
    return peak + np.log(np.exp(y - peak[:, None]).sum(axis=1))


def cross_entropy(logits, labels):
    """Return (loss[M], grad[M, N], lse[M]) in fp64 from fp64 logits."""
    y = np.asarray(logits, dtype=np.float64)
    if y.ndim != 2:
        raise ValueError("logits must be [M, N]")
    n_rows, n_cols = y.shape
    target = np.asarray(labels).astype(np.int64).reshape(n_rows)
    lse = logsumexp_rows(y)
    probs = np.exp(y - lse[:, None])                 # softmax, row by row
    hit = np.flatnonzero((target >= 0) & (target < n_cols))
    picked = np.full(n_rows, np.nan)                 # y[m, label[m]] where defined
    picked[hit] = y[hit, target[hit]]
    loss = lse - picked
    grad = probs.copy()
    grad[hit, target[hit]] -= 1.0                    # minus the one-hot row
    return loss, grad, lse


def tile_partials(logits, tile_edges):
    """Per column tile [tile_edges[t], tile_edges[t+1]): (m_t, s_t) per row.

    Returns two arrays of shape [n_tiles, M].  An empty tile yields the merge
    identity (-inf, 0).
    """
    y = np.asarray(logits, dtype=np.float64)
    M = y.shape[0]
    edges = list(tile_edges)
    ms, ss = [], []
    for lo, hi in zip(edges[:-1], edges[1:]):
        if hi <= lo:
            ms.append(np.full(M, -np.inf))
            ss.append(np.zeros(M))
            continue
        blk = y[:, lo:hi]
        m = blk.max(axis=1)
        ms.append(m)
        ss.append(np.exp(blk - m[:, None]).sum(axis=1))
    return np.array(ms), np.array(ss)


def merge_pair(m1, s1, m2, s2):
    """(m1, s1) (+) (m2, s2) -> (max, s1*exp(m1-max) + s2*exp(m2-max)).

    A side with s == 0 is the identity and is skipped, so -inf - (-inf) is
    never evaluated.
    """
    m1, s1, m2, s2 = (np.asarray(v, dtype=np.float64) for v in (m1, s1, m2, s2))
    mx = np.maximum(m1, m2)
    with np.errstate(invalid="ignore"):
        t1 = np.where(s1 > 0, s1 * np.exp(np.where(s1 > 0, m1 - mx, 0.0)), 0.0)
        t2 = np.where(s2 > 0, s2 * np.exp(np.where(s2 > 0, m2 - mx, 0.0)), 0.0)
    m = np.where(s1 > 0, np.where(s2 > 0, mx, m1), m2)
    return m, t1 + t2


def merge_partials(ms, ss, order=None):
    """Fold [n_tiles, M] partials in ``order`` (default: ascending tiles).

    Returns (m, s, lse) per row, lse = m + log(s).
    """
    ms = np.asarray(ms, dtype=np.float64)
    ss = np.asarray(ss, dtype=np.float64)
    n_tiles, M = ms.shape
    order = range(n_tiles) if order is None else order
    m = np.full(M, -np.inf)
    s = np.zeros(M)
    for t in order:
        m, s = merge_pair(m, s, ms[t], ss[t])
    with np.errstate(divide="ignore"):
        lse = m + np.log(s)
    return m, s, lse
