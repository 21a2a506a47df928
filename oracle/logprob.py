"""Selected-token log-probability over the vocabulary (oracle side).

[RLK] section 4 ("The Shared Dependency of Attention and Linear LogP on
LogSumExp"): LSE(x) = log sum_i exp(x_i), evaluated stably as
m + log sum_i exp(x_i - m) with m the maximum; a token's log-probability is
its logit minus the LSE over the whole vocabulary; when the vocabulary is
split into blocks with local statistics (m_j, s_j), two blocks merge as

    m = max(m1, m2),   s = s1 * exp(m1 - m) + s2 * exp(m2 - m),

and the merge order is part of the contract. [RLK] section 7 (LogP on ROCm):
each shard computes local statistics and they are merged in a fixed
vocabulary-tile order. [VeXact] Eq. (1) defines the per-token mismatch as
the difference of the two sides' log-probabilities.

Readings taken: C chunks with chunk j = [floor(j V / C), floor((j+1) V / C));
the merge order is the balanced tree over chunks; a target id outside
[0, V) yields NaN.

``logprob`` is the plain definition in float64. ``chunk_stats`` and
``merge_tree`` evaluate the chunked form in float64 (equal to the plain form
up to float64 rounding); they localise errors and pin the merge formula.
The GPU's fp32 exp2 / sum order inside a chunk is hardware-defined: bitwise
parity there is UNPINNED, bounded by the 1e-5 relative tolerance.
"""

import numpy as np

from .tree import BALANCED, combine


def chunk_bounds(V, C):
    return [((j * V) // C, ((j + 1) * V) // C) for j in range(C)]


def logprob(logits, target, rows=None):
    """lp[m] = x[m, t_m] - LSE(x[m, :]) in float64."""
    x = np.asarray(logits, dtype=np.float64)
    t = np.asarray(target).astype(np.int64)
    if rows is not None:
        x = x[rows]
        t = t[rows]
    M, V = x.shape
    m = x.max(axis=1)
    lse = m + np.log(np.sum(np.exp(x - m[:, None]), axis=1))
    ok = (t >= 0) & (t < V)
    tl = np.where(ok, x[np.arange(M), np.clip(t, 0, V - 1)], np.nan)
    return tl - lse


def lse(logits):
    x = np.asarray(logits, dtype=np.float64)
    m = x.max(axis=1)
    return m + np.log(np.sum(np.exp(x - m[:, None]), axis=1))


def chunk_stats(logits, C):
    """(m_j, s_j) per row and chunk in float64, arrays [M, C]."""
    x = np.asarray(logits, dtype=np.float64)
    M, V = x.shape
    ms = np.empty((M, C))
    ss = np.empty((M, C))
    for j, (a, b) in enumerate(chunk_bounds(V, C)):
        blk = x[:, a:b]
        ms[:, j] = blk.max(axis=1)
        ss[:, j] = np.sum(np.exp(blk - ms[:, j:j + 1]), axis=1)
    return ms, ss


def merge(a, b):
    """The two-block LSE merge on (m, s) pairs; (-inf, 0) is the identity."""
    m1, s1 = a
    m2, s2 = b
    m = np.maximum(m1, m2)
    with np.errstate(invalid="ignore"):
        f1 = np.where(m1 == -np.inf, 0.0, np.exp(m1 - m))
        f2 = np.where(m2 == -np.inf, 0.0, np.exp(m2 - m))
    return m, s1 * f1 + s2 * f2


def merge_tree(ms, ss, schedule=BALANCED):
    """LSE per row from chunk statistics merged over the given schedule."""
    items = [(ms[:, j], ss[:, j]) for j in range(ms.shape[1])]
    m, s = combine(items, merge, schedule)
    return m + np.log(s)
