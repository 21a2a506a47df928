"""K-leaf GEMM on the GPU: parity with the oracle and bitwise invariance.

IsoExec blog, "Parallelism-invariant kernels": contiguous K leaves, FP32
accumulation per leaf, a binary combine schedule fixed by the contract, and a
fixed rank-to-leaf mapping. RL-Kernel write-up, section 2: two summation
orders of the same values can round differently (the tree-shape pin).
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import gemm as ogemm
from oracle import tree as otree
from split_invariant_deterministic_amd import synth
from tests.helpers import bitwise_equal, check_bf16, check_fp32_gemm, mismatch_report

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DEV = "cuda"


@pytest.fixture(scope="module")
def inv():
    from split_invariant_deterministic_amd import inv as m
    return m


def _np(t):
    return t.float().cpu().numpy()


# ------------------------------------------------------------ oracle parity

@pytest.mark.parametrize("out", ["bf16", "fp32"])
def test_tiny_against_oracle(inv, out):
    t = synth.tiny(0)
    A, B = t["x"].to(DEV), t["W"].to(DEV)
    C = inv.gemm(A, B, inv.contract(leaves=4, out=out))
    ref = ogemm.gemm_tree(_np(t["x"]), _np(t["W"]), 4, out)
    if out == "bf16":
        check_bf16(C, ref, "tiny bf16")
    else:
        check_fp32_gemm(C, ref, "tiny fp32")


@pytest.mark.parametrize("M,N,K,L", [(8, 512, 256, 4), (100, 300, 1024, 8), (33, 17, 512, 8),
                                     (130, 129, 256, 2), (64, 64, 64, 1),
                                     # leaves of 96 (an odd multiple of 32): the fused launch runs them
                                     # as 32-wide substeps of 64-k stages, the per-leaf launches on
                                     # 32-k stages
                                     (200, 300, 768, 8), (150, 200, 384, 4), (130, 129, 192, 2)])
def test_leaf_partials_bound_and_bit_exact_replay(inv, M, N, K, L):
    A = synth.randn((M, K), 101)
    B = synth.randn((N, K), 102, 0.02)
    Ad, Bd = A.to(DEV), B.to(DEV)
    c32 = inv.contract(leaves=L, out="fp32")
    P = inv.gemm_leaves(Ad, Bd, 0, L, c32)
    C32 = inv.gemm(Ad, Bd, c32)
    C16 = inv.gemm(Ad, Bd, inv.contract(leaves=L, out="bf16"))
    Ph = P.cpu().numpy()
    # each GPU leaf sum is within Higham's bound of the exact leaf sum
    An, Bn = _np(A).astype(np.float64), _np(B).astype(np.float64)
    kl = K // L
    for l in range(L):
        exact = An[:, l * kl:(l + 1) * kl] @ Bn[:, l * kl:(l + 1) * kl].T
        absum = np.abs(An[:, l * kl:(l + 1) * kl]) @ np.abs(Bn[:, l * kl:(l + 1) * kl]).T
        assert np.all(np.abs(Ph[l] - exact) <= ogemm.leaf_error_bound(kl, absum)), l
    # the oracle's fp32 tree over the GPU's own partials reproduces the GPU bit for bit
    replay = ogemm.combine_partials(Ph)
    assert np.array_equal(replay.view(np.uint32), C32.cpu().numpy().view(np.uint32))
    r16 = ogemm.cast_out(replay, "bf16").astype(np.float32)
    assert np.array_equal(r16, C16.float().cpu().numpy())
    # and the whole result agrees with the oracle's schedule
    check_fp32_gemm(C32, ogemm.gemm_tree(An, Bn, L, "fp32"), "fp32 vs oracle")
    check_bf16(C16, ogemm.gemm_tree(An, Bn, L, "bf16"), "bf16 vs oracle")


@pytest.mark.parametrize("L", [1, 2, 4, 8])
def test_integer_inputs_are_exact(inv, L):
    """Small integers times powers of two: every summation order is exact."""
    g = torch.Generator().manual_seed(7)
    A = torch.randint(-8, 9, (77, 512), generator=g).to(torch.bfloat16)
    B = (torch.randint(-8, 9, (200, 512), generator=g) * 0.25).to(torch.bfloat16)
    C = inv.gemm(A.to(DEV), B.to(DEV), inv.contract(leaves=L, out="fp32"))
    exact = A.double() @ B.double().T
    assert torch.equal(C.cpu().double(), exact)


def test_tree_shape_pin(inv):
    """Leaves (1, 2^24, 1, -2^24): balanced tree 1.0, left fold 0.0 (stored case)."""
    g = json.load(open(os.path.join(GOLDEN, "tree_order.json")))
    r = g["gemm_realisation"]
    A = torch.zeros((1, r["K"]), dtype=torch.bfloat16)
    B = torch.zeros((16, r["K"]), dtype=torch.bfloat16)
    for k, v in r["A"].items():
        A[0, int(k)] = v
    for k, v in r["B"].items():
        B[0, int(k)] = v
    Ad, Bd = A.to(DEV), B.to(DEV)
    c = inv.contract(leaves=r["leaves"], out="fp32")
    P = inv.gemm_leaves(Ad, Bd, 0, 4, c)
    assert P[:, 0, 0].cpu().tolist() == g["leaves"]
    assert inv.gemm(Ad, Bd, c)[0, 0].item() == g["balanced"]
    fold = inv.tree_combine(P, inv.contract(leaves=4, out="fp32", tree="left_fold"))
    assert fold[0, 0].item() == g["left_fold"]
    bal = inv.tree_combine(P, c)
    assert bal[0, 0].item() == g["balanced"]


@pytest.mark.parametrize("count", [2, 8, 16, 32])
@pytest.mark.parametrize("shape", [(5, 12), (3, 7), (64, 4100)])
def test_tree_combine_against_oracle(inv, count, shape):
    """inv_tree_combine against the oracle's fp32 tree and boundary cast, bit
    for bit, for both trees and both output types, on planes of 60, 21 and
    262400 elements. Partials mix magnitudes over 2^-20 .. 2^20 so that the
    order of the adds decides bits."""
    M, N = shape
    rng = np.random.default_rng(count * 1000 + M)
    P = (rng.standard_normal((count, M, N)) * np.exp2(rng.integers(-20, 21, (count, M, N)))).astype(np.float32)
    Pd = torch.from_numpy(P).to(DEV)
    for tree in ("balanced", "left_fold"):
        for out in ("fp32", "bf16"):
            c = inv.contract(leaves=count, out=out, tree=tree)
            want = ogemm.cast_out(ogemm.combine_partials(P, tree), out)
            got = inv.tree_combine(Pd, c).float().cpu().numpy()
            assert np.array_equal(got.astype(np.float64).view(np.uint64),
                                  np.asarray(want, dtype=np.float64).view(np.uint64)), (tree, out)


# ------------------------------------------------------------ invariance

DENSE = [(4096, 12288), (12288, 4096)]


@pytest.fixture(scope="module")
def dense_inputs():
    out = {}
    for K, N in DENSE:
        d = synth.dense(K, N, M=4096, seed=0, device=DEV)
        out[(K, N)] = (d["X"], d["W"])
    return out


@pytest.mark.parametrize("K,N", DENSE)
def test_dense_batch_invariance_and_sampled_oracle(inv, dense_inputs, K, N):
    X, W = dense_inputs[(K, N)]
    c = inv.contract(leaves=8)
    full = inv.gemm(X, W, c)
    for M in (1, 7, 16, 17, 63, 64, 65, 128, 200, 512):
        part = inv.gemm(X[:M].contiguous(), W, c)
        n, bad, dmax = mismatch_report(part, full[:M])
        assert bad == 0, f"M={M}: {bad}/{n} mismatches, max {dmax}"
        # without the optional workspace: the single-pass kernel, same bits
        assert bitwise_equal(inv.gemm(X[:M].contiguous(), W, c, use_ws=False), part), M
    # rows in another order give the same rows
    perm = torch.randperm(512, generator=torch.Generator().manual_seed(3)).to(DEV)
    pm = inv.gemm(X[perm].contiguous(), W, c)
    assert bitwise_equal(pm, full[perm])
    # sampled rows/columns against the oracle at the full size
    rows = np.array([0, 1, 6, 7, 63, 64, 511, 512, 2047, 4095])
    cols = np.sort(np.random.default_rng(5).choice(N, 96, replace=False))
    Xs = X[torch.as_tensor(rows, device=DEV)].float().cpu().numpy()
    Ws = W[torch.as_tensor(cols, device=DEV)].float().cpu().numpy()
    ref = ogemm.gemm_tree(Xs, Ws, 8, "bf16")
    got = full[torch.as_tensor(rows, device=DEV)][:, torch.as_tensor(cols, device=DEV)]
    check_bf16(got, ref, f"dense {K}->{N} sampled")


@pytest.mark.parametrize("K,N", DENSE)
@pytest.mark.parametrize("M", [7, 33, 512])
def test_rank_partitions_are_bitwise_equal(inv, dense_inputs, K, N, M):
    X, W = dense_inputs[(K, N)]
    X = X[:M].contiguous()
    base = inv.gemm(X, W, inv.contract(leaves=8, ranks=1))
    for R in (2, 4, 8):
        c = inv.contract(leaves=8, ranks=R)
        assert bitwise_equal(inv.gemm(X, W, c), base), f"ranks={R}"
        # explicit per-rank launches, nothing transported, then the pinned top of the tree
        P = torch.stack([inv.gemm_rank(X, W, r, c) for r in range(R)])
        assert bitwise_equal(inv.tree_combine(P, c), base), f"gemm_rank ranks={R}"
    # per-leaf launches replayed by the combine
    P8 = inv.gemm_leaves(X, W, 0, 8, inv.contract(leaves=8, out="fp32"))
    assert bitwise_equal(inv.tree_combine(P8, inv.contract(leaves=8)), base)


@pytest.mark.parametrize("M", [65, 300])
def test_odd_leaf_rank_partitions_are_bitwise_equal(inv, M):
    """K = 768, 8 leaves of 96: ranks 1, 2 and 4 run their leaves as 32-wide
    substeps of 64-k stages, ranks 8 (one leaf a launch) on 32-k stages; the
    chain per element is the same, so the bits are."""
    X = synth.randn((M, 768), 111).to(DEV)
    W = synth.randn((256, 768), 112, 0.02).to(DEV)
    base = inv.gemm(X, W, inv.contract(leaves=8, ranks=1))
    for R in (2, 4, 8):
        c = inv.contract(leaves=8, ranks=R)
        P = torch.stack([inv.gemm_rank(X, W, r, c) for r in range(R)])
        assert bitwise_equal(inv.tree_combine(P, c), base), f"gemm_rank ranks={R}"
    P8 = inv.gemm_leaves(X, W, 0, 8, inv.contract(leaves=8, out="fp32"))
    assert bitwise_equal(inv.tree_combine(P8, inv.contract(leaves=8)), base)


@pytest.mark.parametrize("M,N,K,out", [(1100, 3900, 512, "bf16"), (1000, 4100, 1024, "fp32"), (2048, 2100, 768, "bf16")])
def test_many_tiles_ragged(inv, M, N, K, out):
    """More output tiles than resident workgroups, ragged in rows and columns:
    every row is bitwise the same row computed in a small launch, and sampled
    elements match the oracle's tree."""
    X = synth.randn((M, K), 121).to(DEV)
    W = synth.randn((N, K), 122, 0.02).to(DEV)
    c = inv.contract(leaves=8, out=out)
    full = inv.gemm(X, W, c)
    for r0, r1 in ((0, 100), (M - 77, M), (512, 640)):
        part = inv.gemm(X[r0:r1].contiguous(), W, c)
        n, bad, dmax = mismatch_report(part, full[r0:r1])
        assert bad == 0, f"rows {r0}:{r1}: {bad}/{n} mismatches, max {dmax}"
    rows = np.array([0, 127, 128, 513, M - 1])
    cols = np.sort(np.random.default_rng(7).choice(N, 64, replace=False))
    cols[-1] = N - 1
    Xs = X[torch.as_tensor(rows, device=DEV)].float().cpu().numpy()
    Ws = W[torch.as_tensor(cols, device=DEV)].float().cpu().numpy()
    ref = ogemm.gemm_tree(Xs, Ws, 8, out)
    got = full[torch.as_tensor(rows, device=DEV)][:, torch.as_tensor(cols, device=DEV)]
    if out == "bf16":
        check_bf16(got, ref, f"{M}x{N}x{K} sampled")
    else:
        check_fp32_gemm(got, ref, f"{M}x{N}x{K} sampled")


def test_left_fold_changes_bits(inv, dense_inputs):
    """Teeth: a different combine schedule must move some bits."""
    X, W = dense_inputs[(4096, 12288)]
    X = X[:64].contiguous()
    P = inv.gemm_leaves(X, W, 0, 8, inv.contract(leaves=8, out="fp32"))
    bal = inv.tree_combine(P, inv.contract(leaves=8, out="fp32"))
    fold = inv.tree_combine(P, inv.contract(leaves=8, out="fp32", tree="left_fold"))
    n, bad, _ = mismatch_report(bal, fold)
    assert bad > 0
    assert bitwise_equal(bal, inv.gemm(X, W, inv.contract(leaves=8, out="fp32")))


def test_repeat_runs_are_bitwise_stable(inv, dense_inputs):
    X, W = dense_inputs[(12288, 4096)]
    c = inv.contract(leaves=8)
    first = inv.gemm(X, W, c)
    for _ in range(20):
        assert bitwise_equal(inv.gemm(X, W, c), first)


def test_empty_and_ragged(inv):
    c = inv.contract(leaves=8)
    A = torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)
    B = synth.randn((40, 256), 9).to(DEV)
    assert inv.gemm(A, B, c).shape == (0, 40)
    A = synth.randn((65, 256), 10).to(DEV)  # one row past the small-M kernel
    full = inv.gemm(A, B, c)
    for M in (1, 16, 17, 64):
        assert bitwise_equal(inv.gemm(A[:M].contiguous(), B, c), full[:M]), M


@pytest.mark.parametrize("M", [9, 300, 2100])
def test_leaves_of_32_rank_partitions_and_oracle(inv, M):
    """K = 256, 8 leaves of 32 k: one MFMA step per leaf, on 32-k stages for
    every leaf count; rank partitions and per-leaf launches give the bits of
    the single launch, and sampled elements match the oracle."""
    X = synth.randn((M, 256), 141).to(DEV)
    W = synth.randn((2000, 256), 142, 0.05).to(DEV)
    base = inv.gemm(X, W, inv.contract(leaves=8))
    assert bitwise_equal(inv.gemm(X, W, inv.contract(leaves=8), use_ws=False), base)
    for R in (2, 4, 8):
        assert bitwise_equal(inv.gemm(X, W, inv.contract(leaves=8, ranks=R)), base), R
    P8 = inv.gemm_leaves(X, W, 0, 8, inv.contract(leaves=8, out="fp32"))
    assert bitwise_equal(inv.tree_combine(P8, inv.contract(leaves=8)), base)
    rows = np.array([0, M // 2, M - 1])
    ref = ogemm.gemm_tree(X[torch.as_tensor(rows, device=DEV)].float().cpu().numpy(), W.float().cpu().numpy(), 8, "bf16")
    check_bf16(base[torch.as_tensor(rows, device=DEV)], ref, f"leaves of 32, M={M}")


@pytest.mark.parametrize("M,N,K,out", [(9, 1000, 1024, "bf16"), (40, 515, 2048, "fp32"), (64, 130, 512, "bf16"),
                                       (33, 16400, 1024, "fp32")])  # 129 column tiles x 2 groups: persistent
def test_small_m_64_row_tiles(inv, M, N, K, out):
    """8 <= M <= 64 runs on 64-row tiles (8 waves of 64 x 16), persistent when
    the (column tile, leaf group) items outnumber the CUs. Ragged columns,
    leaf groups, emulated ranks and per-leaf launches all give the bits of the
    128-row tiles (the same rows inside a 65-row launch), and the result
    matches the oracle element by element. The last case's ranks 4 and 8
    walk 516 and 1032 persistent items of 4 and 2 stages, fewer than the
    5-stage ring holds: every stage of an item is issued before the item's
    own turn sets up its successor (the issue side then switches tiles at
    that set-up)."""
    X = synth.randn((65, K), 151).to(DEV)
    W = synth.randn((N, K), 152, 0.02).to(DEV)
    c = inv.contract(leaves=8, out=out)
    big = inv.gemm(X, W, c)  # 65 rows: 128-row tiles
    Xm = X[:M].contiguous()
    base = inv.gemm(Xm, W, c, use_ws=False)
    assert bitwise_equal(base, big[:M])
    assert bitwise_equal(inv.gemm(Xm, W, c), base)  # with the leaf-group workspace
    for R in (2, 4, 8):
        assert bitwise_equal(inv.gemm(Xm, W, inv.contract(leaves=8, ranks=R, out=out)), base), R
    P8 = inv.gemm_leaves(Xm, W, 0, 8, inv.contract(leaves=8, out="fp32"))
    assert bitwise_equal(inv.tree_combine(P8, c), base)
    ref = ogemm.gemm_tree(Xm.float().cpu().numpy(), W.float().cpu().numpy(), 8, out)
    if out == "bf16":
        check_bf16(base, ref, f"64-row tiles M={M} N={N} K={K}")
    else:
        check_fp32_gemm(base, ref, f"64-row tiles M={M} N={N} K={K}")
