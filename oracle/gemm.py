"""K-leaf GEMM (oracle side).

[IsoExec] "Parallelism-invariant kernels" / [NovaSky] "Making kernels
parallelism-invariant": the contraction dimension K is cut into contiguous
leaves; each leaf is accumulated with FP32 accumulation; the leaf partials
are combined in FP32 by a binary schedule fixed by the contract, with a fixed
rank-to-leaf mapping. [RLK] section 7 (GEMM on ROCm): fixed chunk order,
merge in FP32, write BF16 once.

Notation: A [M, K] activations, B [N, K] the weight stored K-contiguous (the
pages' "K x N" weight, transposed in storage only), L leaves, leaf l covering
k in [l*K/L, (l+1)*K/L).

What is computed here:

* ``leaf_partials``: P_l = fp32( sum_k A[m,k] * B[n,k] ) with the sum taken in
  float64. Products of two bf16 values are exact in float64 and the float64
  sum error is far below one fp32 ulp, so P_l is the fp32 rounding of a
  near-exact sum. The GPU's per-leaf MFMA chain rounds differently inside the
  leaf (hardware-defined): bitwise parity of single leaves is UNPINNED and is
  checked by the error bound ``leaf_error_bound`` instead.
* ``combine_partials``: the fp32 tree over partials, replayed bit-exactly
  (numpy float32 adds are IEEE RNE without contraction). Fed the GPU's own
  partials it must reproduce the GPU's output bit for bit.
* ``gemm``: the plain definition C = round_out(sum over all K in float64),
  and ``gemm_tree``: the leaf/tree schedule with float64 leaves.
* ``exact_leaf_sums``: exact rational sums (``fractions.Fraction``) for tiny
  inputs, used to pin ``leaf_partials``.
"""

from fractions import Fraction

import numpy as np

from . import numerics
from .tree import BALANCED, combine


def _leaf_bounds(K, leaves):
    if leaves <= 0 or K % leaves != 0:
        raise ValueError("K must be a multiple of the leaf count")
    kl = K // leaves
    return [(l * kl, (l + 1) * kl) for l in range(leaves)]


def leaf_partials(A, B, leaves, leaf_lo=0, leaf_hi=None, rows=None, cols=None):
    """fp32 leaf partials P [leaf_hi-leaf_lo, M', N'] (float32).

    ``rows`` / ``cols`` select a subset of output rows / columns (for sampled
    checks at full size); the arithmetic per element is unchanged.
    """
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    if rows is not None:
        A = A[rows]
    if cols is not None:
        B = B[cols]
    K = A.shape[1]
    bounds = _leaf_bounds(K, leaves)
    if leaf_hi is None:
        leaf_hi = leaves
    out = np.empty((leaf_hi - leaf_lo, A.shape[0], B.shape[0]), dtype=np.float32)
    for i, l in enumerate(range(leaf_lo, leaf_hi)):
        k0, k1 = bounds[l]
        out[i] = numerics.f32(A[:, k0:k1] @ B[:, k0:k1].T)
    return out


def combine_partials(P, schedule=BALANCED):
    """fp32 tree over the leading axis of P (float32 adds, bit-exact replay)."""
    P = np.asarray(P, dtype=np.float32)
    return combine([P[i] for i in range(P.shape[0])], lambda a, b: (a + b).astype(np.float32),
                   schedule)


def cast_out(C32, out_dtype):
    """Boundary cast of fp32 values: 'bf16' (RNE, returned as float64 values) or 'fp32'."""
    if out_dtype == "bf16":
        return numerics.to_bf16(np.asarray(C32, dtype=np.float32).astype(np.float64))
    if out_dtype == "fp32":
        return np.asarray(C32, dtype=np.float32)
    raise ValueError(out_dtype)


def gemm_tree(A, B, leaves, out_dtype="bf16", schedule=BALANCED, rows=None, cols=None):
    """The leaf/tree rounding schedule with float64 leaf sums."""
    P = leaf_partials(A, B, leaves, rows=rows, cols=cols)
    return cast_out(combine_partials(P, schedule), out_dtype)


def gemm(A, B, out_dtype="bf16", rows=None, cols=None):
    """Plain definition: C = round_out( sum_k A[m,k] B[n,k] ) in float64."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    if rows is not None:
        A = A[rows]
    if cols is not None:
        B = B[cols]
    C = A @ B.T
    if out_dtype == "bf16":
        return numerics.to_bf16(C)
    if out_dtype == "fp64":
        return C
    return numerics.f32(C)


def abs_products(A, B, leaves, rows=None, cols=None):
    """sum_k |A[m,k]| |B[n,k]| per leaf, float64 [L, M', N'] (for error bounds)."""
    A = np.abs(np.asarray(A, dtype=np.float64))
    B = np.abs(np.asarray(B, dtype=np.float64))
    if rows is not None:
        A = A[rows]
    if cols is not None:
        B = B[cols]
    K = A.shape[1]
    return np.stack([A[:, k0:k1] @ B[:, k0:k1].T for k0, k1 in _leaf_bounds(K, leaves)])


def leaf_error_bound(n_terms, abs_sum, u=2.0 ** -24):
    """Higham's gamma_n bound for any fp32 summation order of n_terms exact
    products: |computed - exact| <= n*u/(1-n*u) * sum|a b|, plus one rounding."""
    n = float(n_terms)
    return (n * u / (1.0 - n * u)) * abs_sum + u * abs_sum


def exact_leaf_sums(A, B, leaves):
    """Exact rational leaf sums [L][M][N] of Fractions (tiny inputs only)."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    M, K = A.shape
    N = B.shape[0]
    Af = [[Fraction(float(A[m, k])) for k in range(K)] for m in range(M)]
    Bf = [[Fraction(float(B[n, k])) for k in range(K)] for n in range(N)]
    out = []
    for k0, k1 in _leaf_bounds(K, leaves):
        out.append([[sum((Af[m][k] * Bf[n][k] for k in range(k0, k1)), Fraction(0))
                     for n in range(N)] for m in range(M)])
    return out
