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

LM-head schedule (the fused GEMM + logprob): blocks of a fixed width of 16
columns, block b = [16 b, min(16 b + 16, V)), merged by the balanced tree
over the block index after padding the block list with the identity
(-inf, 0) to a power of two (for a power-of-two count this is the same tree
as ``merge_tree``; for other counts the padding fixes where the short
subtree sits). ``block_stats`` and ``merge_tree_padded`` write it out.

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


def _stats(blk):
    """(max, sum of exp(x - max)) per row of a block. An element equal to -inf
    adds exactly 0, so a block whose elements are all -inf (a masked range of
    the vocabulary) is the merge identity (-inf, 0) rather than NaN."""
    m = blk.max(axis=1)
    with np.errstate(invalid="ignore"):
        e = np.where(blk == -np.inf, 0.0, np.exp(blk - m[:, None]))
    return m, np.sum(e, axis=1)


def chunk_stats(logits, C):
    """(m_j, s_j) per row and chunk in float64, arrays [M, C]."""
    x = np.asarray(logits, dtype=np.float64)
    M, V = x.shape
    ms = np.empty((M, C))
    ss = np.empty((M, C))
    for j, (a, b) in enumerate(chunk_bounds(V, C)):
        ms[:, j], ss[:, j] = _stats(x[:, a:b])
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


def block_bounds(V, width=16):
    """Fixed-width vocabulary blocks [w b, min(w b + w, V))."""
    return [(a, min(a + width, V)) for a in range(0, V, width)]


def block_stats(logits, width=16):
    """(m_b, s_b) per row and fixed-width block in float64, arrays [M, nb]."""
    x = np.asarray(logits, dtype=np.float64)
    M, V = x.shape
    bounds = block_bounds(V, width)
    ms = np.empty((M, len(bounds)))
    ss = np.empty((M, len(bounds)))
    for j, (a, b) in enumerate(bounds):
        ms[:, j], ss[:, j] = _stats(x[:, a:b])
    return ms, ss


def pad_pow2(items, identity):
    """items followed by copies of identity up to the next power of two."""
    P = 1
    while P < len(items):
        P *= 2
    return list(items) + [identity] * (P - len(items))


def merge_tree_padded(ms, ss):
    """LSE per row: balanced tree over the blocks padded with (-inf, 0) to 2^k."""
    M, n = ms.shape
    items = pad_pow2([(ms[:, j], ss[:, j]) for j in range(n)], (np.full(M, -np.inf), np.zeros(M)))
    m, s = combine(items, merge, BALANCED)
    return m + np.log(s)


def logprob_blocks(logits, target, width=16):
    """lp through the block schedule, float64 (equals ``logprob`` up to rounding)."""
    x = np.asarray(logits, dtype=np.float64)
    t = np.asarray(target).astype(np.int64)
    M, V = x.shape
    lse_ = merge_tree_padded(*block_stats(x, width))
    ok = (t >= 0) & (t < V)
    tl = np.where(ok, x[np.arange(M), np.clip(t, 0, V - 1)], np.nan)
    return tl - lse_
