"""Gated DeltaNet under the chunkwise-parallel recurrent (CPR) schedule (oracle side).

[IsoExec] "Chunkwise-parallel recurrent (CPR) GDN" and [NovaSky] "Solving the
linear-attention headache": Gated DeltaNet's chunk-parallel form (used for
training and prefill) and its token-recurrent form (used for decode) compute
the same function but round differently. Under CPR the token recurrence is
the definition. Prefill obtains the state at each multiple of the chunk size
with a separate pass and then evaluates every chunk's tokens independently,
starting from that chunk's opening state. Decode steps the recurrence token
by token and, each time a chunk completes, replaces its running state with
the chunk-boundary state, so prefill, training forward and decode follow one
rounding schedule. [IsoExec] "Unified execution contract" lists gdn.core,
gdn.gating and norms.l2 among its example regions.

The pages give no formulas for the layer. Readings taken (the gated delta
rule of Gated DeltaNet, restated; one head, key and value width 128):

    k^_t = k_t / sqrt(sum k_t^2 + eps),  q^_t = q_t / sqrt(sum q_t^2 + eps) / sqrt(d_k)
    alpha_t = exp(g_t)  (g_t <= 0 is the given log-decay),  beta_t in [0, 1] given
    S_t = alpha_t (S_{t-1} - beta_t k^_t (k^_t^T S_{t-1})) + beta_t k^_t v_t^T,   S_0 = 0
    o_t = S_t^T q^_t

with eps = 1e-6, S of shape [d_k, d_v]. The boundary states use the
chunkwise closed form of the same recurrence (derived from it by unrolling
over a chunk; ``chunk_update``), with gamma_t the running product of alpha
inside the chunk:

    w_t = beta_t (v_t - gamma_t S_0^T k^_t - sum_{s<t} (gamma_t / gamma_s) (k^_s . k^_t) w_s)
    S_C = gamma_C S_0 + sum_s (gamma_C / gamma_s) k^_s w_s^T

Boundaries sit at multiples of the chunk size C counted from each sequence's
first token; a sequence of length L has boundary states b_0 = 0, ..., b_n
with n = floor(L / C), and the tokens of chunk j are evaluated by the
recurrence from b_j.

Everything here is float64. ``recurrent`` is the plain definition;
``chunk_update`` and ``cpr`` are the closed form and the CPR schedule, equal
to it up to float64 rounding (pinned in tests). The GPU's fp32 rounding inside
a chunk update and inside the recurrence steps is hardware/implementation
defined: bitwise parity with the oracle is UNPINNED there; the GPU is pinned
against itself (prefill = decode, bit for bit) and against this oracle within
a tolerance.
"""

import numpy as np

EPS = 1e-6


def l2norm(x, eps=EPS):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def prep(q, k, g):
    """(q^, k^, alpha) of the definition above; the last axis is the head width."""
    q = np.asarray(q, dtype=np.float64)
    dk = q.shape[-1]
    return l2norm(q) / np.sqrt(dk), l2norm(k), np.exp(np.asarray(g, dtype=np.float64))


def recurrent(qh, kh, v, alpha, beta, S0=None):
    """Token-by-token recurrence for one head: o [L, dv], final state [dk, dv]."""
    kh = np.asarray(kh, dtype=np.float64)
    qh = np.asarray(qh, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L, dk = kh.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.empty((L, dv))
    for t in range(L):
        a, b = float(alpha[t]), float(beta[t])
        S = a * (S - b * np.outer(kh[t], kh[t] @ S)) + b * np.outer(kh[t], v[t])
        o[t] = S.T @ qh[t]
    return o, S


def chunk_update(S0, kh, v, alpha, beta):
    """State after one chunk by the closed form (unrolled recurrence)."""
    kh = np.asarray(kh, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    C = kh.shape[0]
    gamma = np.cumprod(np.asarray(alpha, dtype=np.float64))
    P = kh @ S0                       # S_0^T k^_t for every t, as rows
    w = np.empty_like(v)
    for t in range(C):
        acc = v[t] - gamma[t] * P[t]
        for s in range(t):
            acc = acc - (gamma[t] / gamma[s]) * (kh[s] @ kh[t]) * w[s]
        w[t] = float(beta[t]) * acc
    c = gamma[-1] / gamma
    return gamma[-1] * S0 + (kh * c[:, None]).T @ w


def cpr(qh, kh, v, alpha, beta, C):
    """CPR schedule for one head of one sequence.

    Returns (o [L, dv], boundaries [n+1, dk, dv], running state after the
    last token): boundary b_{j+1} = chunk_update(b_j, chunk j); outputs of
    chunk j by the recurrence from b_j. When L is a multiple of C the running
    state is the last boundary (the state decode switches to there)."""
    kh = np.asarray(kh, dtype=np.float64)
    L, dk = kh.shape
    dv = np.asarray(v).shape[1]
    n = L // C
    b = [np.zeros((dk, dv))]
    for j in range(n):
        sl = slice(j * C, (j + 1) * C)
        b.append(chunk_update(b[-1], kh[sl], v[sl], alpha[sl], beta[sl]))
    o = np.empty((L, dv))
    run = b[n]
    for j in range((L + C - 1) // C):
        sl = slice(j * C, min((j + 1) * C, L))
        o[sl], S = recurrent(qh[sl], kh[sl], v[sl], alpha[sl], beta[sl], b[j])
        if j == n:
            run = S
    return o, np.stack(b), run


def gdn_layer(q, k, v, g, beta, cu_seqlens, C):
    """All heads of packed sequences: q, k, v [T, H, 128], g, beta [T, H].

    Returns o [T, H, 128] float64 through the CPR schedule."""
    qh, kh, alpha = prep(q, k, g)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T, H, _ = kh.shape
    o = np.empty(v.shape)
    for s in range(len(cu_seqlens) - 1):
        a, e = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        for h in range(H):
            o[a:e, h], _, _ = cpr(qh[a:e, h], kh[a:e, h], v[a:e, h], alpha[a:e, h], beta[a:e, h], C)
    return o
