"""Pins of the CPU oracle against facts it does not compute itself.

Each test ties one oracle function to something independent: a closed form,
an exact rational computation, a hand-computed case from the pages' own
examples, a textbook library routine, or an invariant. A plausible mistake
in the oracle (a dropped term, a wrong index or sign, a transposed operand,
a wrong tree) fails at least one of them. These run on the CPU only.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import gdn as ogdn
from oracle import gemm as ogemm
from oracle import logprob as olp
from oracle import moe as omoe
from oracle import numerics
from oracle import rmsnorm as orms
from oracle import tree as otree
from split_invariant_deterministic_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 cast

def _stratified_f32_bits(n_random=1 << 18, seed=0):
    rng = np.random.default_rng(seed)
    r = rng.integers(0, 1 << 32, size=n_random, dtype=np.uint64).astype(np.uint32)
    hi = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    # every exponent/sign/mantissa-high pattern with the low half at and next
    # to the rounding midpoint, plus exact bf16 values
    lows = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    edge = (hi[:, None] | lows[None, :]).ravel()
    return np.concatenate([r, edge])


def test_bf16_cast_matches_torch_rne():
    bits = _stratified_f32_bits()
    f = bits.view(np.float32)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns
        ours = numerics.to_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(f)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].astype(np.float32).view(np.uint32),
                          ref[~nan].view(np.uint32))


def test_bf16_hand_ties():
    one = 1.0
    assert numerics.to_bf16(one + 2.0 ** -8) == 1.0            # tie -> even (mantissa 0)
    assert numerics.to_bf16(one + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6  # tie -> even (mantissa 2)
    assert numerics.to_bf16(one + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert numerics.to_bf16(-0.0) == 0.0 and math.copysign(1, numerics.to_bf16(-0.0)) < 0
    assert numerics.to_bf16(3.5e38) == np.inf
    assert numerics.to_bf16(2.0 ** -133) == 2.0 ** -133          # smallest subnormal
    assert numerics.to_bf16(2.0 ** -134) == 0.0                  # tie -> even zero


# ---------------------------------------------------------------- tree shape

def test_tree_schedules_hand_case():
    g = json.load(open(os.path.join(GOLDEN, "tree_order.json")))
    leaves = [np.float32(v) for v in g["leaves"]]
    add = lambda a, b: np.float32(a + b)
    assert otree.combine(leaves, add, otree.BALANCED) == np.float32(g["balanced"])
    assert otree.combine(leaves, add, otree.LEFT_FOLD) == np.float32(g["left_fold"])


def test_tree_shape_through_gemm_oracle():
    g = json.load(open(os.path.join(GOLDEN, "tree_order.json")))
    r = g["gemm_realisation"]
    A = np.zeros((1, r["K"]))
    B = np.zeros((1, r["K"]))
    for k, v in r["A"].items():
        A[0, int(k)] = v
    for k, v in r["B"].items():
        B[0, int(k)] = v
    P = ogemm.leaf_partials(A, B, r["leaves"])
    assert P[:, 0, 0].tolist() == g["leaves"]
    assert ogemm.gemm_tree(A, B, 4, "fp32")[0, 0] == g["balanced"]
    assert ogemm.gemm_tree(A, B, 4, "fp32", otree.LEFT_FOLD)[0, 0] == g["left_fold"]
    assert ogemm.gemm_tree(A, B, 4, "bf16")[0, 0] == 1.0
    # the plain definition sees the exact sum 1 + 2**24 + 1 - 2**24 = 2
    assert ogemm.gemm(A, B, "fp32")[0, 0] == 2.0


def test_balanced_is_adjacent_pairs_for_powers_of_two():
    # recursive halving == pairing (0,1),(2,3),... level by level
    names = [f"x{i}" for i in range(8)]
    s = otree.balanced(names, lambda a, b: f"({a}+{b})")
    assert s == "(((x0+x1)+(x2+x3))+((x4+x5)+(x6+x7)))"
    # every aligned 2-, 4-block is a subtree (rank-local reduction is possible)
    for blk in ("(x0+x1)", "(x6+x7)", "((x0+x1)+(x2+x3))", "((x4+x5)+(x6+x7))"):
        assert blk in s


# ---------------------------------------------------------------- GEMM leaves

def test_leaf_sums_against_exact_rationals():
    t = synth.tiny()
    A = t["x"].float().numpy()
    B = t["W"].float().numpy()[:48]  # 48 output columns keep Fraction work small
    P = ogemm.leaf_partials(A, B, 4)
    ex = ogemm.exact_leaf_sums(A, B, 4)
    absp = ogemm.abs_products(A, B, 4)
    for l in range(4):
        for m in range(A.shape[0]):
            for n in range(B.shape[0]):
                e = ex[l][m][n]
                err = abs(Fraction(float(P[l, m, n])) - e)
                # half an fp32 ulp of the exact value plus the float64 sum error
                bound = Fraction(2.0 ** -24) * abs(e) + Fraction(64 * 2.0 ** -53) * Fraction(absp[l, m, n])
                assert err <= bound, (l, m, n)


def test_leaf_partition_covers_k_and_tree_matches_plain_sum():
    t = synth.tiny()
    A = t["x"].float().numpy()
    B = t["W"].float().numpy()
    P = ogemm.leaf_partials(A, B, 4)
    # a wrong leaf range (gap/overlap/transposed operand) breaks this identity
    exact = A.astype(np.float64) @ B.astype(np.float64).T
    assert np.allclose(P.astype(np.float64).sum(0), exact, rtol=0, atol=1e-5)
    C = ogemm.combine_partials(P)
    bound = ogemm.leaf_error_bound(64 + 2, ogemm.abs_products(A, B, 1)[0])
    assert np.all(np.abs(C.astype(np.float64) - exact) <= bound)


def test_integer_valued_gemm_is_exact_for_every_schedule():
    rng = np.random.default_rng(1)
    A = rng.integers(-8, 9, size=(5, 256)).astype(np.float64)
    B = rng.integers(-8, 9, size=(7, 256)).astype(np.float64) * 0.25
    exact = A @ B.T  # every partial sum < 2**24: all orders exact
    for leaves in (1, 2, 4, 8):
        for sch in (otree.BALANCED, otree.LEFT_FOLD):
            assert np.array_equal(ogemm.gemm_tree(A, B, leaves, "fp32", sch), exact.astype(np.float32))


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_closed_forms():
    H = 256
    g = np.ones(H)
    assert np.all(orms.rmsnorm(np.zeros((1, H)), g) == 0.0)
    assert np.all(orms.rmsnorm(np.ones((1, H)), g) == 1.0)        # 1/sqrt(1+eps) -> 1.0
    x = np.zeros((1, H))
    x[0, 17] = 1.0
    y = orms.rmsnorm(x, g)
    assert y[0, 17] == 16.0 and np.count_nonzero(y) == 1          # sqrt(256)*(1-1.3e-4) -> 16
    # gamma multiplies per column, sign carries through
    gg = np.linspace(-2, 2, H)
    y2 = orms.rmsnorm(np.ones((1, H)) * -3.0, gg)
    assert np.array_equal(y2[0], numerics.to_bf16(-gg / math.sqrt(1 + np.float32(1e-6) / 9)))


def test_rmsnorm_sum_of_squares_exact_on_tiny():
    x = synth.tiny()["x"].float().numpy().astype(np.float64)
    eps = float(np.float32(1e-6))
    for m in range(x.shape[0]):
        ss = sum((Fraction(float(v)) ** 2 for v in x[m]), Fraction(0))
        r_exact = 1.0 / math.sqrt(float(ss / x.shape[1]) + eps)
        assert abs(orms.inv_rms(x[m:m + 1])[0] - r_exact) <= 4e-16 * r_exact


# ---------------------------------------------------------------- logprob

def test_logprob_constant_logits_is_minus_log_v():
    g = json.load(open(os.path.join(GOLDEN, "logprob_constant.json")))
    V = g["V"]
    x = np.full((3, V), g["value"])
    lp = olp.logprob(x, np.array([0, 5, V - 1]))
    assert np.allclose(lp, g["expected"], rtol=0, atol=1e-15)
    ms, ss = olp.chunk_stats(x, g["chunks"])
    assert np.all(ss == g["chunk_sum"]) and np.all(ms == g["value"])


def test_logprob_matches_torch_log_softmax_and_normalises():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(6, 300)) * 3
    t = rng.integers(0, 300, size=6)
    ref = torch.log_softmax(torch.from_numpy(x), dim=-1).numpy()
    assert np.allclose(olp.logprob(x, t), ref[np.arange(6), t], rtol=0, atol=1e-13)
    all_t = np.stack([olp.logprob(x, np.full(6, v)) for v in range(300)], 1)
    assert np.allclose(np.exp(all_t).sum(1), 1.0, rtol=0, atol=1e-12)


def test_logprob_chunked_tree_equals_plain_lse():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(4, 2374 * 3 + 5)) * 2
    for C in (1, 2, 4, 64):
        ms, ss = olp.chunk_stats(x, C)
        for sch in (otree.BALANCED, otree.LEFT_FOLD):
            assert np.allclose(olp.merge_tree(ms, ss, sch), olp.lse(x), rtol=0, atol=1e-12)


def test_block_schedule_partitions_and_equals_plain_lse():
    """The 16-column block schedule of the fused LM head: blocks tile [0, V),
    and block statistics merged over the padded tree give the plain LSE."""
    rng = np.random.default_rng(14)
    for V in (1, 15, 16, 17, 100, 1000, 2374 * 3 + 5):
        b = olp.block_bounds(V)
        assert b[0][0] == 0 and b[-1][1] == V
        assert all(hi - lo == 16 for lo, hi in b[:-1]) and 1 <= b[-1][1] - b[-1][0] <= 16
        assert all(b[i][1] == b[i + 1][0] for i in range(len(b) - 1))
        x = rng.normal(size=(3, V)) * 3
        assert np.allclose(olp.merge_tree_padded(*olp.block_stats(x)), olp.lse(x), rtol=0, atol=1e-12)
        t = np.array([0, V - 1, V])
        lp = olp.logprob_blocks(x, t)
        assert np.allclose(lp[:2], olp.logprob(x, t)[:2], rtol=0, atol=1e-12) and np.isnan(lp[2])


def test_padded_tree_shape():
    """Padding to a power of two fixes the tree for any block count: five
    blocks pair as ((0,1),(2,3)),(4,pad) -- not the ceil-halving tree
    ((0,1),2),(3,4) -- and the padding merges away exactly."""
    cat = lambda a, b: f"({a}{b})"
    assert otree.combine(olp.pad_pow2(list("abcde"), "_"), cat) == "(((ab)(cd))((e_)(__)))"
    assert otree.combine(list("abcde"), cat) == "(((ab)c)(de))"
    assert olp.pad_pow2(list("abcd"), "_") == list("abcd")
    # the identity is exact in the merge, so a padded tree equals its unpadded twin
    rng = np.random.default_rng(15)
    ms, ss = rng.normal(size=(2, 8)), rng.uniform(1, 16, size=(2, 8))
    full = olp.merge_tree(ms, ss)
    assert np.array_equal(olp.merge_tree_padded(ms, ss), full)


def test_lse_merge_identity_and_halves():
    m, s = np.array([0.7]), np.array([3.25])
    mi, si = olp.merge((np.array([-np.inf]), np.array([0.0])), (m, s))
    assert mi[0] == m[0] and si[0] == s[0]
    mh, sh = olp.merge((m, s), (m, s))
    assert mh[0] == m[0] and sh[0] == 2 * s[0]
    # the merge is the LSE of the union
    x = np.array([[0.1, 2.0, -1.0, 0.5, 3.0]])
    a = (np.array([2.0]), np.array([np.exp(0.1 - 2) + 1 + np.exp(-3)]))
    b = (np.array([3.0]), np.array([np.exp(0.5 - 3) + 1]))
    mm, ssum = olp.merge(a, b)
    assert abs(mm[0] + np.log(ssum[0]) - olp.lse(x)[0]) < 1e-14


def test_chunk_bounds_floor_rule_hand_values():
    """Chunk j = [floor(jV/C), floor((j+1)V/C)): hand-derived boundaries that
    the other plausible splits (ceil-first as numpy.array_split, remainder to
    the last chunk) get wrong."""
    assert olp.chunk_bounds(10, 4) == [(0, 2), (2, 5), (5, 7), (7, 10)]
    # the LM-head vocabulary: 151936 = 64 * 2374, every chunk 2374 long
    b = olp.chunk_bounds(151936, 64)
    assert [e - a for a, e in b] == [2374] * 64 and b[-1] == (151936 - 2374, 151936)
    # one logit more: floor((j+1)(64*2374+1)/64) - floor(j(64*2374+1)/64) = 2374 + [j = 63]
    assert [e - a for a, e in olp.chunk_bounds(151937, 64)] == [2374] * 63 + [2375]
    # one logit less: only chunk 0 is short (floor(-1/64) = -1)
    assert [e - a for a, e in olp.chunk_bounds(151935, 64)] == [2373] + [2374] * 63
    # the statistics follow the same boundaries: zero logits give s_j = chunk length
    ms, ss = olp.chunk_stats(np.zeros((1, 10)), 4)
    assert ss[0].tolist() == [2.0, 3.0, 2.0, 3.0] and np.all(ms == 0.0)


def test_masked_chunks_are_the_merge_identity():
    """A chunk whose logits are all -inf (a masked vocabulary range) has the
    statistics (-inf, 0), the exact identity of the merge, so the chunked LSE
    equals the plain one; scattered -inf entries add exactly nothing."""
    rng = np.random.default_rng(21)
    x = rng.normal(size=(3, 40))
    x[0, 10:20] = -np.inf          # chunk 1 of 4 fully masked
    x[1, ::3] = -np.inf            # scattered
    x[2, 30:40] = -np.inf
    x[2, 0:10] = -np.inf
    ms, ss = olp.chunk_stats(x, 4)
    assert ms[0, 1] == -np.inf and ss[0, 1] == 0.0
    assert ms[2, 0] == -np.inf and ss[2, 0] == 0.0 and ss[2, 3] == 0.0
    assert not np.any(np.isnan(ss))
    for sch in (otree.BALANCED, otree.LEFT_FOLD):
        assert np.allclose(olp.merge_tree(ms, ss, sch), olp.lse(x), rtol=0, atol=1e-13)
    # the plain value: the masked entries drop out of the sum
    keep = np.isfinite(x[1])
    assert abs(olp.lse(x)[1] - np.log(np.sum(np.exp(x[1][keep])))) < 1e-13
    bm, bs = olp.block_stats(x)
    assert not np.any(np.isnan(bs))
    assert np.allclose(olp.merge_tree_padded(bm, bs), olp.lse(x), rtol=0, atol=1e-13)
    t = np.array([5, 1, 25])
    assert np.allclose(olp.logprob_blocks(x, t), olp.logprob(x, t), rtol=0, atol=1e-13)


def test_logprob_bad_target_is_nan():
    x = np.zeros((3, 10))
    lp = olp.logprob(x, np.array([-1, 10, 3]))
    assert np.isnan(lp[0]) and np.isnan(lp[1]) and not np.isnan(lp[2])


# ---------------------------------------------------------------- attention

def _attn_case(lengths, Hq=8, Hkv=2, D=16, seed=5):
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q = numerics.to_bf16(rng.normal(size=(len(lengths), Hq, D)))
    k = numerics.to_bf16(rng.normal(size=(cu[-1], Hkv, D)))
    v = numerics.to_bf16(rng.normal(size=(cu[-1], Hkv, D)))
    return q, k, v, cu, np.arange(len(lengths)), lengths - 1


def test_split_bounds_partition_the_visible_keys():
    for L in (1, 2, 15, 16, 17, 63, 64, 65, 1023, 1024, 1025, 32768, 5000):
        b = oatt.split_bounds(L, 16, 64)
        assert b[0][0] == 0 and b[-1][1] == L
        for (a0, a1), (c0, c1) in zip(b, b[1:]):
            assert a1 == c0 and a0 <= a1
        for a, e in b:
            assert a % 64 == 0 or a == L
    # one chunk: only the last split is non-empty
    assert [a < e for a, e in oatt.split_bounds(40, 16, 64)] == [False] * 15 + [True]


def test_attention_single_key_returns_v0():
    q, k, v, cu, qs, qp = _attn_case([1, 1])
    out = oatt.attention(q, k, v, cu, qs, qp, 2)
    for i in range(2):
        for h in range(8):
            assert np.array_equal(out[i, h], v[cu[i], h // 4])


def test_attention_equal_keys_is_mean_of_v():
    q, k, v, cu, qs, qp = _attn_case([37])
    k[:] = k[0]
    out = oatt.attention(q, k, v, cu, qs, qp, 2)
    for h in range(8):
        assert np.array_equal(out[0, h], numerics.to_bf16(v[:, h // 4].mean(0)))


def test_attention_matches_torch_sdpa_float64():
    q, k, v, cu, qs, qp = _attn_case([5, 130, 64])
    out = oatt.attention(q, k, v, cu, qs, qp, 2, round_bf16=False)
    for i in range(3):
        kk = torch.from_numpy(k[cu[i]:cu[i] + qp[i] + 1]).permute(1, 0, 2).repeat_interleave(4, 0)
        vv = torch.from_numpy(v[cu[i]:cu[i] + qp[i] + 1]).permute(1, 0, 2).repeat_interleave(4, 0)
        qq = torch.from_numpy(q[i]).unsqueeze(1)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[:, 0].numpy()
        assert np.allclose(out[i], ref, rtol=0, atol=1e-12)


def test_attention_split_states_merge_to_plain():
    q, k, v, cu, qs, qp = _attn_case([1, 3, 64, 65, 700, 1025], seed=6)
    plain = oatt.attention(q, k, v, cu, qs, qp, 2, round_bf16=False)
    for S, ch in ((1, 64), (4, 32), (16, 64)):
        for sch in (otree.BALANCED, otree.LEFT_FOLD):
            got = oatt.attention_splits(q, k, v, cu, qs, qp, 2, S, ch, sch)
            assert np.allclose(got, plain, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- MoE

def test_route_matches_torch_topk_and_ties():
    rng = np.random.default_rng(7)
    x = rng.normal(size=(20, 128))
    ids, w = omoe.route(x, 8)
    top = torch.topk(torch.from_numpy(x), 8, dim=1).indices.numpy()
    assert np.array_equal(ids, np.sort(top, axis=1))
    z = np.take_along_axis(x, ids, 1)
    assert np.allclose(w, np.exp(z) / np.exp(z).sum(1, keepdims=True), atol=1e-7)
    ids2, w2 = omoe.route(np.zeros((2, 16)), 4)
    assert ids2.tolist() == [[0, 1, 2, 3]] * 2 and np.all(w2 == 0.25)
    x3 = np.zeros((1, 16))
    x3[0, [3, 9, 12]] = 5.0
    x3[0, [1, 2]] = 1.0
    x3[0, [0, 4]] = 1.0  # 0,1,2,4 tie at 1.0: lower ids win
    ids3, _ = omoe.route(x3, 5)
    assert ids3[0].tolist() == [0, 1, 3, 9, 12]


def test_swiglu_closed_forms():
    gu = np.array([[0.0, 2.0, 1.0, 1.0], [-60.0, 30.0, 3.0, 0.5]])
    a = omoe.swiglu(gu)
    assert a[0, 0] == 0.0                                   # silu(0) = 0
    assert a[0, 1] == numerics.to_bf16(2.0 / (1 + math.exp(-2.0)))
    assert a[1, 0] == numerics.to_bf16(-60.0 / (1 + math.exp(60.0)) * 3.0)
    assert a[1, 1] == 15.0                                  # silu(30) = 30 (to bf16), * 0.5


def test_moe_identical_experts_equal_one_expert():
    rng = np.random.default_rng(8)
    T, H, F, E = 6, 64, 32, 16
    x = numerics.to_bf16(rng.normal(size=(T, H)))
    W1 = numerics.to_bf16(rng.normal(size=(2 * F, H)) * 0.1)
    W2 = numerics.to_bf16(rng.normal(size=(H, F)) * 0.1)
    out, ids, w = omoe.moe_layer(x, np.zeros((T, E)), np.stack([W1] * E), np.stack([W2] * E), 8)
    assert np.all(w == 0.125) and ids.tolist() == [list(range(8))] * T
    single = numerics.to_bf16(omoe.expert_ffn(x, W1, W2).astype(np.float64))
    assert np.array_equal(out, single)


def _rne_rational(q, bits):
    """Round an exact rational to the nearest value with ``bits`` significant
    bits (8: bf16, 24: fp32), ties to even, computed on the rational itself
    (normal range only; these tests stay far from over- and underflow)."""
    if q == 0:
        return 0.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2**e <= a < 2**(e+2)
    if a < Fraction(2) ** e:
        e -= 1
    elif a >= Fraction(2) ** (e + 1):
        e += 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1) and -120 < e < 120
    ulp = Fraction(2) ** (e - bits + 1)
    n = a / ulp
    f = n.numerator // n.denominator
    r = n - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return float((f * ulp) if q > 0 else -(f * ulp))


def test_rne_rational_helper_hand_cases():
    # the helper itself, on hand-checked values
    assert _rne_rational(Fraction(1) + Fraction(1, 256), 8) == 1.0              # tie -> even
    assert _rne_rational(Fraction(1) + Fraction(3, 256), 8) == 1.0 + 2.0 ** -6  # tie -> even (up)
    assert _rne_rational(Fraction(-3, 7), 24) == float(np.float32(-3.0 / 7.0))
    assert _rne_rational(Fraction(1, 3), 8) == 0.333984375                       # 0x3EAB


def test_moe_gate_up_and_down_against_exact_rationals():
    """gate_up = bf16(x W1^T) and down = fp32(a W2^T) on a non-square shape
    (x 3x24, W1 10x24, W2 24x5): every entry is the exact rational sum
    rounded once at the boundary. A transposed operand fails on the shapes, a
    dropped boundary rounding or a wrong index on the values."""
    gen = torch.Generator().manual_seed(31)
    x = torch.randn(3, 24, generator=gen).to(torch.bfloat16).double().numpy()
    W1 = (torch.randn(10, 24, generator=gen) * 0.3).to(torch.bfloat16).double().numpy()
    W2 = (torch.randn(24, 5, generator=gen) * 0.3).to(torch.bfloat16).double().numpy()
    gu = omoe.gate_up(x, W1)
    assert gu.shape == (3, 10)
    for i in range(3):
        for j in range(10):
            ex = sum((Fraction(float(x[i, k])) * Fraction(float(W1[j, k])) for k in range(24)), Fraction(0))
            assert gu[i, j] == _rne_rational(ex, 8), (i, j)
    a = omoe.swiglu(gu)
    assert a.shape == (3, 5)
    y = omoe.down(a, W2)
    assert y.shape == (3, 24) and y.dtype == np.float32
    for i in range(3):
        for h in range(24):
            ex = sum((Fraction(float(a[i, f])) * Fraction(float(W2[h, f])) for f in range(5)), Fraction(0))
            assert float(y[i, h]) == _rne_rational(ex, 24), (i, h)
    # the rounding is really exercised: the unrounded sums differ from the results
    assert not np.array_equal(gu, x @ W1.T) and not np.array_equal(y.astype(np.float64), a @ W2.T)


def test_moe_ffn_integer_closed_form():
    """Small integers: g, u, a and y are exact, so gate_up is the integer
    product, the SwiGLU of g = 0 is 0, and down reproduces a W2^T exactly."""
    rng = np.random.default_rng(32)
    x = rng.integers(-3, 4, size=(4, 24)).astype(np.float64)
    W1 = rng.integers(-2, 3, size=(10, 24)).astype(np.float64)
    gu = omoe.gate_up(x, W1)
    assert np.array_equal(gu, x @ W1.T)          # |entries| <= 144 < 256: bf16-exact
    a = rng.integers(-4, 5, size=(4, 5)).astype(np.float64)
    W2 = rng.integers(-4, 5, size=(24, 5)).astype(np.float64)
    assert np.array_equal(omoe.down(a, W2), (a @ W2.T).astype(np.float32))
    gz = np.concatenate([np.zeros((2, 5)), np.ones((2, 5)) * 7.0], axis=1)
    assert np.all(omoe.swiglu(gz) == 0.0)       # silu(0) * u = 0


# ---------------------------------------------------------------- Gated DeltaNet (CPR)

def _gdn_case(L, dk=16, dv=12, seed=0, gscale=0.2):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(L, dk))
    k = rng.normal(size=(L, dk))
    v = rng.normal(size=(L, dv))
    g = -gscale * rng.uniform(size=L)
    beta = rng.uniform(size=L)
    qh, kh, alpha = ogdn.prep(q, k, g)
    return qh, kh, v, alpha, beta


def test_gdn_chunk_closed_form_equals_the_recurrence():
    """The boundary-state closed form is the recurrence unrolled over a chunk."""
    for C, seed in ((1, 1), (2, 2), (5, 3), (16, 4), (64, 5)):
        qh, kh, v, alpha, beta = _gdn_case(C, seed=seed)
        S0 = np.random.default_rng(seed + 10).normal(size=(16, 12))
        _, S = ogdn.recurrent(qh, kh, v, alpha, beta, S0)
        assert np.allclose(ogdn.chunk_update(S0, kh, v, alpha, beta), S, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,C", [(1, 4), (7, 4), (64, 16), (100, 16), (130, 64)])
def test_gdn_cpr_equals_the_recurrence(L, C):
    qh, kh, v, alpha, beta = _gdn_case(L, seed=L)
    o_ref, S_ref = ogdn.recurrent(qh, kh, v, alpha, beta)
    o, b, run = ogdn.cpr(qh, kh, v, alpha, beta, C)
    assert b.shape[0] == L // C + 1 and not b[0].any()
    assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
    assert np.allclose(run, S_ref, rtol=0, atol=1e-12)
    for j in range(1, L // C + 1):   # every boundary is the recurrence's state there
        _, Sj = ogdn.recurrent(qh[:j * C], kh[:j * C], v[:j * C], alpha[:j * C], beta[:j * C])
        assert np.allclose(b[j], Sj, rtol=0, atol=1e-12)


def test_gdn_layer_packed_equals_per_sequence_recurrence():
    """gdn_layer over packed ragged sequences (lengths 1, 63, 64, 65, 130;
    2 heads; chunk 64 and 16) equals, per sequence and head, the plain token
    recurrence run on that sequence alone from a zero state; the order in
    which sequences are packed does not change any sequence's outputs."""
    lengths = [1, 63, 64, 65, 130]
    rng = np.random.default_rng(33)
    T, H, D = sum(lengths), 2, 16
    q = rng.normal(size=(T, H, D))
    k = rng.normal(size=(T, H, D))
    v = rng.normal(size=(T, H, D))
    g = -0.5 * rng.uniform(size=(T, H))
    beta = rng.uniform(size=(T, H))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    for C in (64, 16):
        o = ogdn.gdn_layer(q, k, v, g, beta, cu, C)
        assert o.shape == (T, H, D)
        for s in range(len(lengths)):
            a, e = cu[s], cu[s + 1]
            for h in range(H):
                qh, kh, al = ogdn.prep(q[a:e, h], k[a:e, h], g[a:e, h])
                ref, _ = ogdn.recurrent(qh, kh, v[a:e, h], al, beta[a:e, h])
                assert np.allclose(o[a:e, h], ref, rtol=0, atol=1e-12), (C, s, h)
    # reversed packing order: same per-sequence outputs
    order = list(range(len(lengths)))[::-1]
    idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in order])
    cu2 = np.concatenate([[0], np.cumsum([lengths[s] for s in order])])
    o2 = ogdn.gdn_layer(q[idx], k[idx], v[idx], g[idx], beta[idx], cu2, 64)
    assert np.allclose(o2, ogdn.gdn_layer(q, k, v, g, beta, cu, 64)[idx], rtol=0, atol=1e-12)


def test_gdn_delta_rule_closed_forms():
    dk, dv = 8, 5
    rng = np.random.default_rng(9)
    vals = rng.normal(size=(dk, dv))
    eye = np.eye(dk)
    # beta = 1, no decay, orthonormal keys: each write stores its value exactly
    kh, alpha, beta = eye, np.ones(dk), np.ones(dk)
    _, S = ogdn.recurrent(np.zeros((dk, dk)), kh, vals, alpha, beta)
    assert np.allclose(S, vals, rtol=0, atol=1e-15)
    # a second write to the same unit key replaces the first (the delta rule); with a key of
    # squared norm n the old value survives as (1 - n) n v1 (what l2norm's eps leaves)
    k1 = rng.normal(size=dk)
    k1 = k1 / np.linalg.norm(k1)
    v1, v2 = rng.normal(size=dv), rng.normal(size=dv)
    _, S = ogdn.recurrent(np.zeros((2, dk)), np.stack([k1, k1]), np.stack([v1, v2]), np.ones(2), np.ones(2))
    assert np.allclose(S.T @ k1, v2, rtol=0, atol=1e-12)
    k2 = ogdn.l2norm(rng.normal(size=(1, dk)))[0]
    n = k2 @ k2
    _, S = ogdn.recurrent(np.zeros((2, dk)), np.stack([k2, k2]), np.stack([v1, v2]), np.ones(2), np.ones(2))
    assert np.allclose(S.T @ k2, n * v2 + (1 - n) * n * v1, rtol=0, atol=1e-14) and n < 1
    # beta = 0: nothing is written, the zero state stays zero and outputs are exact zeros
    qh, kh, v, alpha, _ = _gdn_case(20)
    o, S = ogdn.recurrent(qh, kh, v, alpha, np.zeros(20))
    assert not o.any() and not S.any()
    # pure decay of one write: S_t = (prod alpha) k v^T
    a = np.array([1.0, 0.5, 0.25, 0.8])
    _, S = ogdn.recurrent(np.zeros((4, dk)), np.stack([eye[2]] * 4), np.stack([vals[0]] + [np.zeros(dv)] * 3), a,
                          np.array([1.0, 0.0, 0.0, 0.0]))
    assert np.allclose(S, 0.5 * 0.25 * 0.8 * np.outer(eye[2], vals[0]), rtol=0, atol=1e-15)
    # the l2 norm and the query scale
    q = np.array([[3.0, 4.0] + [0.0] * 6])
    qh, kh, _ = ogdn.prep(q, q, np.zeros(1))
    assert np.allclose(kh[0, :2], [3 / math.sqrt(25 + 1e-6), 4 / math.sqrt(25 + 1e-6)], rtol=1e-15)
    assert np.allclose(qh, kh / math.sqrt(8), rtol=1e-15)


# ---------------------------------------------------------------- generator

def test_synth_tiny_is_fixed_per_seed():
    g = json.load(open(os.path.join(GOLDEN, "synth_hashes.json")))
    t = synth.tiny(0)
    import hashlib
    for name in ("x", "W", "targets"):
        h = hashlib.sha256(t[name].contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()
        assert h == g[name], name


def test_oracle_reproduces_stored_tiny_values():
    """Regression pin: a later change to the oracle's arithmetic must be deliberate."""
    g = np.load(os.path.join(GOLDEN, "tiny_expected.npz"))
    t = synth.tiny(0)
    y = orms.rmsnorm(t["x"].float().numpy(), t["gamma"].float().numpy(), 1e-6)
    assert np.array_equal(y.astype(np.float32), g["rms_y"])
    lt = ogemm.gemm_tree(y, t["W"].float().numpy(), 4, "fp32")
    assert np.array_equal(lt, g["logits_tree"])
    assert np.array_equal(olp.logprob(lt, t["targets"].numpy()), g["logprob"])
