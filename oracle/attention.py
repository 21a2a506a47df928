"""Attention over visible keys with a pinned split rule (oracle side).

[RLK] section 4: attention softmax is a reduction over the visible key range
and shares the LSE statistic and its two-block merge with the vocabulary
log-softmax. [IsoExec] "Unified execution contract": split-KV partition
counts are pinned constants of the composition. [RLK] section 7: the
optional ROCm attention path fixes the block partition, the chunk order and
the rescale-merge order.

``attention`` is the plain definition in float64,

    out[i, h] = bf16( softmax( q[i,h] . K^T / sqrt(D) ) V ),

over keys [0, q_pos[i]] of the row's sequence, query head h reading kv head
h // (Hq / Hkv).

``split_bounds`` is the split rule (a reading, since the pages give only the
count): keys form chunks of ``kv_chunk`` from position 0, a row with L
visible keys has n = ceil(L / kv_chunk) chunks, and split j of S owns chunks
[floor(j n / S), floor((j+1) n / S)). ``attention_splits`` evaluates each
split's (m, l, o) in float64 and merges them with the same schedule and the
LSE merge extended to o (o scaled like l); in exact arithmetic this equals
the plain definition, which pins the split bookkeeping. The GPU's rounding
inside a split (bf16 p, MFMA chains) is hardware-defined: bitwise parity is
UNPINNED, bounded by one bf16 ulp against the plain definition.
"""

import math

import numpy as np

from . import numerics
from .tree import BALANCED, combine


def split_bounds(L, split_kv, kv_chunk):
    """Key ranges [a, b) of each split for a row with L visible keys."""
    n = -(-L // kv_chunk)
    out = []
    for j in range(split_kv):
        c0 = (j * n) // split_kv
        c1 = ((j + 1) * n) // split_kv
        out.append((min(c0 * kv_chunk, L), min(c1 * kv_chunk, L)))
    return out


def _row_keys(k, v, cu_seqlens, seq, pos, g):
    start = int(cu_seqlens[seq])
    keys = np.asarray(k[start:start + pos + 1, g, :], dtype=np.float64)
    vals = np.asarray(v[start:start + pos + 1, g, :], dtype=np.float64)
    return keys, vals


def attention(q, k, v, cu_seqlens, q_seq, q_pos, Hkv, round_bf16=True):
    """Plain attention per (row, head); float64, rounded to bf16 at the end."""
    q = np.asarray(q, dtype=np.float64)
    Tq, Hq, D = q.shape
    grp = Hq // Hkv
    out = np.empty((Tq, Hq, D))
    scale = 1.0 / math.sqrt(D)
    for i in range(Tq):
        for g in range(Hkv):
            keys, vals = _row_keys(k, v, cu_seqlens, int(q_seq[i]), int(q_pos[i]), g)
            s = q[i, g * grp:(g + 1) * grp, :] @ keys.T * scale  # [grp, L]
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            out[i, g * grp:(g + 1) * grp, :] = (p @ vals) / p.sum(axis=1, keepdims=True)
    return numerics.to_bf16(out) if round_bf16 else out


def _merge_state(a, b):
    m1, l1, o1 = a
    m2, l2, o2 = b
    m = max(m1, m2)
    if m == -math.inf:
        return a
    f1 = 0.0 if m1 == -math.inf else math.exp(m1 - m)
    f2 = 0.0 if m2 == -math.inf else math.exp(m2 - m)
    return m, l1 * f1 + l2 * f2, o1 * f1 + o2 * f2


def attention_splits(q, k, v, cu_seqlens, q_seq, q_pos, Hkv, split_kv, kv_chunk,
                     schedule=BALANCED):
    """float64 split states merged by the schedule; returns float64 out."""
    q = np.asarray(q, dtype=np.float64)
    Tq, Hq, D = q.shape
    grp = Hq // Hkv
    scale = 1.0 / math.sqrt(D)
    out = np.empty((Tq, Hq, D))
    for i in range(Tq):
        L = int(q_pos[i]) + 1
        bounds = split_bounds(L, split_kv, kv_chunk)
        for h in range(Hq):
            keys, vals = _row_keys(k, v, cu_seqlens, int(q_seq[i]), int(q_pos[i]), h // grp)
            states = []
            for a, b in bounds:
                if a >= b:
                    states.append((-math.inf, 0.0, np.zeros(D)))
                    continue
                s = keys[a:b] @ q[i, h] * scale
                m = float(s.max())
                p = np.exp(s - m)
                states.append((m, float(p.sum()), p @ vals[a:b]))
            m, l, o = combine(states, _merge_state, schedule)
            out[i, h] = o / l
    return out
