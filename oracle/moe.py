"""Mixture-of-experts layer: routing, expert FFN, fixed-order combine (oracle side).

[IsoExec] "Unified model": deterministic MoE routing and combination.
[IsoExec] "Parallelism-invariant kernels" / [NovaSky] "Making kernels
parallelism-invariant": under expert parallelism the order in which a token's
expert results are summed is tied to the routing, never to which rank
produced them. [IsoExec] "Unified execution contract": the moe.combine
region is pinned to a leaf tree with 8 leaves of fp32. [RLK] sections 6 and 7
(FFN module): packed gate/up GEMM, SwiGLU and down GEMM run as separate,
fixed stages.

Readings taken (the pages give no formulas for these steps):

* routing: the k largest router logits, ties resolved toward the lower expert
  id; weights = softmax over the k selected logits; experts listed in
  ascending id;
* SwiGLU with W1 = [gate; up] packed along the output dimension:
  a = silu(g) * u, silu(g) = g / (1 + exp(-g)), g and u taken at their bf16
  boundary, a rounded to bf16;
* down projection output kept in fp32 (the combine's leaf dtype);
* combine: leaves w_j * y_j in fp32 for the token's experts in ascending id,
  fp32 balanced tree, one bf16 rounding.

GEMMs and the softmax are the plain float64 definitions; the fp32 leaf
products and the fp32 tree are replayed bit-exactly (numpy float32).
Pinned by: torch.topk on tie-free logits, eight identical experts with equal
logits (w = 1/8 exactly, output = one expert's FFN), and hand-made ties.
"""

import numpy as np

from . import numerics
from .tree import BALANCED, combine as tree_combine


def route(logits, k):
    """ids [T, k] int32 ascending, w [T, k] float32 (softmax over the selection)."""
    x = np.asarray(logits, dtype=np.float64)
    T, E = x.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-x[t, e], e))[:k]
        sel = sorted(order)
        z = x[t, sel]
        p = np.exp(z - z.max())
        ids[t] = sel
        w[t] = numerics.f32(p / p.sum())
    return ids, w


def gate_up(x_rows, W1e):
    """[g | u] = bf16( x W1e^T ) in float64; W1e [2F, K]."""
    return numerics.to_bf16(np.asarray(x_rows, np.float64) @ np.asarray(W1e, np.float64).T)


def swiglu(gu):
    """a = bf16( silu(g) * u ), gu = [g | u] of bf16 values."""
    gu = np.asarray(gu, dtype=np.float64)
    F = gu.shape[1] // 2
    g, u = gu[:, :F], gu[:, F:]
    return numerics.to_bf16(g / (1.0 + np.exp(-g)) * u)


def down(a, W2e):
    """y = fp32( a W2e^T ) in float64; W2e [H, F]."""
    return numerics.f32(np.asarray(a, np.float64) @ np.asarray(W2e, np.float64).T)


def combine(y_by_leaf, w, schedule=BALANCED):
    """out = bf16( tree_j fp32(w_j * y_j) ). y_by_leaf [T, k, H] fp32, w [T, k] fp32."""
    y = np.asarray(y_by_leaf, dtype=np.float32)
    w = np.asarray(w, dtype=np.float32)
    leaves = [(w[:, j:j + 1] * y[:, j, :]).astype(np.float32) for j in range(y.shape[1])]
    s = tree_combine(leaves, lambda a, b: (a + b).astype(np.float32), schedule)
    return numerics.to_bf16(s.astype(np.float64))


def expert_ffn(x_rows, W1e, W2e):
    return down(swiglu(gate_up(x_rows, W1e)), W2e)


def moe_layer(x, logits, W1, W2, k, schedule=BALANCED):
    """Full chain in float64 with the pinned boundaries; returns (out, ids, w)."""
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    ids, w = route(logits, k)
    y = np.zeros((T, k, W2.shape[1]), dtype=np.float32)
    for e in np.unique(ids):
        tok, j = np.nonzero(ids == e)
        y[tok, j, :] = expert_ffn(x[tok], W1[e], W2[e])
    return combine(y, w, schedule), ids, w
