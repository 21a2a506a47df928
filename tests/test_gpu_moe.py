"""MoE layer on the GPU: routing, grouping, expert FFN and the fixed-order
combine; oracle parity per stage and bitwise invariance across token splits.

IsoExec blog, "Unified model": deterministic routing and combination;
"Parallelism-invariant kernels": expert outputs combined in a fixed routing
order, not rank order; "Unified execution contract": moe.combine as a tree of
8 fp32 leaves. RL-Kernel write-up, sections 6-7: packed gate/up GEMM, SwiGLU,
down GEMM as separate stages.
"""

import numpy as np
import pytest
import torch

from oracle import moe as omoe
from oracle import numerics
from split_invariant_deterministic_amd import synth
from tests.helpers import bitwise_equal, check_bf16, check_fp32_gemm, mismatch_report

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def inv():
    from split_invariant_deterministic_amd import inv as m
    return m


def _np(t):
    return t.float().cpu().numpy()


def test_route_against_oracle(inv):
    logits = synth.randn((300, 128), 5, dtype=torch.float32)
    ids, w = inv.moe_route(logits.to(DEV), inv.contract(leaves=8))
    oid, ow = omoe.route(logits.double().numpy(), 8)
    assert np.array_equal(ids.cpu().numpy(), oid)
    assert np.allclose(w.cpu().numpy(), ow, rtol=1e-6, atol=0)


def test_route_ties_go_to_lower_ids(inv):
    x = torch.zeros((3, 16))
    x[1, [3, 9, 12]] = 5.0
    x[1, [0, 1, 2, 4]] = 1.0
    x[2] = torch.arange(16, dtype=torch.float32) * 0  # all equal
    ids, w = inv.moe_route(x.to(DEV), inv.contract(leaves=4))
    oid, ow = omoe.route(x.double().numpy(), 4)
    assert np.array_equal(ids.cpu().numpy(), oid)
    assert torch.all(w[0] == 0.25) and torch.all(w[2] == 0.25)
    ids5, _ = inv.moe_route(x[1:2].to(DEV), inv.contract(leaves=2))
    assert ids5.cpu().tolist() == [[3, 9]]


def test_route_signed_zeros_and_minus_inf(inv):
    # -0 and +0 compare equal, so the lower id takes the last slot between
    # them whichever sign it has; -inf logits are selectable (after every
    # finite one) and get weight exactly 0
    x = torch.full((5, 64), -1.0)
    x[0:2, 0:7] = 1.0
    x[0, [10, 50]] = torch.tensor([-0.0, 0.0])
    x[1, [10, 50]] = torch.tensor([0.0, -0.0])
    x[2, :] = float("-inf")
    x[2, [5, 40]] = torch.tensor([0.5, -2.0])      # two finite, then -inf by id
    x[3, :] = float("-inf")
    x[3, 63] = -0.0
    x[4] = torch.randn(64, generator=torch.Generator().manual_seed(7)).round()  # many ties
    ids, w = inv.moe_route(x.to(DEV), inv.contract(leaves=8))
    oid, ow = omoe.route(x.double().numpy(), 8)
    assert np.array_equal(ids.cpu().numpy(), oid)
    assert np.allclose(w.cpu().numpy(), ow, rtol=1e-6, atol=0)
    assert ids[0].cpu().tolist() == [0, 1, 2, 3, 4, 5, 6, 10]
    assert ids[1].cpu().tolist() == [0, 1, 2, 3, 4, 5, 6, 10]
    finite = (ids[2] == 5) | (ids[2] == 40)
    assert (w[2][~finite] == 0).all() and (w[2][finite] > 0).all()


def test_route_nan_rows_are_marked(inv):
    x = torch.randn((2, 16), generator=torch.Generator().manual_seed(1))
    x[0, :13] = float("nan")   # only 3 selectable experts for k = 4
    ids, w = inv.moe_route(x.to(DEV), inv.contract(leaves=4))
    assert (ids[0] == -1).sum().item() == 1 and torch.isnan(w[0]).any()
    assert (ids[1] >= 0).all() and not torch.isnan(w[1]).any()


def _grouping(ids, E):
    k = ids.shape[1]
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    slot = np.empty_like(flat)
    slot[order] = np.arange(len(flat))
    return offsets, order // k, slot.reshape(ids.shape)


def test_permute_is_the_stable_grouping(inv):
    logits = synth.randn((1000, 128), 6, dtype=torch.float32)
    c = inv.contract(leaves=8)
    ids, _ = inv.moe_route(logits.to(DEV), c)
    offsets, rows, slot = inv.moe_permute(ids, 128, c)
    o, r, s = _grouping(ids.cpu().numpy(), 128)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(rows.cpu().numpy(), r)
    assert np.array_equal(slot.cpu().numpy(), s)


class _Experts:
    """Lazy float64 view of a bf16 expert tensor: converts one expert at a time."""

    def __init__(self, W):
        self.W = W
        self.shape = tuple(W.shape)

    def __getitem__(self, e):
        return self.W[int(e)].float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def moe_full():
    return synth.moe(T=8192, seed=0, device=DEV)


def test_moe_stages_against_oracle(inv, moe_full):
    d = moe_full
    T = 96
    x, logits = d["x"][:T].contiguous(), d["logits"][:T].contiguous()
    cg, cr = inv.contract(leaves=8), inv.contract(leaves=8)
    st = {}
    out = inv.moe_layer(x, logits, d["W1"], d["W2"], cg, cr, out_stage=st)
    xn = _np(x).astype(np.float64)
    ids = st["ids"].cpu().numpy()
    oid, ow = omoe.route(logits.double().cpu().numpy(), 8)
    assert np.array_equal(ids, oid)
    rows = st["rows"].cpu().numpy()
    offs = st["offsets"].cpu().numpy()
    W1, W2 = _Experts(d["W1"]), _Experts(d["W2"])
    GU, A, Y = _np(st["GU"]), _np(st["A"]), st["Y"].cpu().numpy()
    for e in np.unique(ids):
        r0, r1 = offs[e], offs[e + 1]
        # each stage consumes the GPU's previous stage (stage-wise parity)
        check_bf16(GU[r0:r1], omoe.gate_up(xn[rows[r0:r1]], W1[e]), f"gate/up e={e}")
        check_bf16(A[r0:r1], omoe.swiglu(GU[r0:r1]), f"swiglu e={e}")
        check_fp32_gemm(Y[r0:r1], omoe.down(A[r0:r1], W2[e]), f"down e={e}")
    # the combine replays bit for bit from the GPU's Y and weights
    slot = st["slot"].cpu().numpy()
    ref = omoe.combine(Y[slot], st["w"].cpu().numpy())
    assert np.array_equal(_np(out), ref.astype(np.float32))
    # free-running chain (information bar: 1 ulp may cascade, so normwise only)
    full, _, _ = omoe.moe_layer(xn, logits.double().cpu().numpy(), W1, W2, 8)
    rel = np.linalg.norm(_np(out) - full) / np.linalg.norm(full)
    assert rel < 2e-2


def test_moe_token_splits_are_bitwise_equal(inv, moe_full):
    d = moe_full
    c = inv.contract(leaves=8)
    full = inv.moe_layer(d["x"], d["logits"], d["W1"], d["W2"], c, c)
    for S in (4, 16):
        n = 8192 // S
        parts = [inv.moe_layer(d["x"][i * n:(i + 1) * n].contiguous(), d["logits"][i * n:(i + 1) * n].contiguous(),
                               d["W1"], d["W2"], c, c) for i in range(S)]
        cnt, bad, dmax = mismatch_report(torch.cat(parts), full)
        assert bad == 0, f"split {S}: {bad}/{cnt}, max {dmax}"
    one = inv.moe_layer(d["x"][4000:4001].contiguous(), d["logits"][4000:4001].contiguous(), d["W1"], d["W2"], c, c)
    assert bitwise_equal(one[0], full[4000])


def test_identical_experts_equal_one_expert(inv):
    """Eight identical experts with equal logits: w = 1/8 exactly and the
    combine returns the single expert's FFN output (oracle pin, GPU side)."""
    T, H, F, E = 40, 256, 256, 16
    x = synth.randn((T, H), 21).to(DEV)
    W1e = synth.randn((2 * F, H), 22, 0.05).to(DEV)
    W2e = synth.randn((H, F), 23, 0.05).to(DEV)
    W1 = W1e.unsqueeze(0).expand(E, 2 * F, H).contiguous()
    W2 = W2e.unsqueeze(0).expand(E, H, F).contiguous()
    c = inv.contract(leaves=8)
    st = {}
    out = inv.moe_layer(x, torch.zeros((T, E), device=DEV), W1, W2, c, c, out_stage=st)
    assert torch.all(st["w"] == 0.125)
    g = inv.gemm(x, W1e, inv.contract(leaves=8))
    a = inv.swiglu(g, c)
    y = inv.gemm(a, W2e, inv.contract(leaves=8, out="fp32"))
    assert bitwise_equal(out, inv.cast_bf16(y))


@pytest.mark.parametrize("T,E,H,F,L", [(96, 128, 2048, 768, 8),   # the layer's shape (96 tokens)
                                         (40, 16, 256, 100, 8),     # ragged F, 32-wide leaves (odd path)
                                         (33, 8, 512, 64, 4),       # one output tile per expert
                                         (7, 4, 128, 200, 1)])      # one leaf, a partial last tile
def test_fused_swiglu_equals_unfused(inv, T, E, H, F, L):
    """The gate/up GEMM with the SwiGLU in its epilogue is bitwise the
    unfused grouped GEMM (bf16 gate/up) followed by the SwiGLU kernel,
    including the NaN rows of malformed gather indices."""
    c = inv.contract(leaves=L)
    x = synth.randn((T, H), 41).to(DEV)
    W1 = synth.randn((E, 2 * F, H), 42, 0.02).to(DEV)
    logits = synth.randn((T, E), 43, dtype=torch.float32).to(DEV)
    k = min(8, E)
    ids, _ = inv.moe_route(logits, inv.contract(leaves=k))
    offsets, rows, _ = inv.moe_permute(ids, E, inv.contract(leaves=k))
    R = T * k
    bad = rows.clone()
    bad[3] = T + 5  # outside [0, T): a NaN row in both paths
    bad[R // 2] = -1
    for rr in (rows, bad):
        fused = inv.moe_gemm_swiglu(x, rr, offsets, W1, R, c)
        ref = inv.swiglu(inv.moe_gemm(x, rr, offsets, W1, R, c), c)
        assert bitwise_equal(fused, ref)
    assert torch.isnan(fused[3]).all() and torch.isnan(fused[R // 2]).all()
    assert not torch.isnan(fused[4]).any()


@pytest.mark.parametrize("out,K,T,E,N", [("fp32", 768, 37, 8, 200), ("bf16", 512, 37, 8, 200), ("fp32", 256, 37, 8, 200),
                                         # more row-tile slots than resident workgroups: each
                                         # workgroup walks several tiles
                                         ("bf16", 512, 600, 16, 2000), ("fp32", 512, 600, 16, 1000),
                                         ("fp32", 768, 600, 16, 2000),
                                         # more than 128 experts: the expert table is searched per tile
                                         ("bf16", 512, 600, 160, 300), ("fp32", 768, 300, 200, 256)])
def test_grouped_gemm_malformed_rows_are_nan(inv, out, K, T, E, N):
    """A gathered index outside [0, x_rows) gives a NaN output row; every other
    row is bitwise the plain K-leaf GEMM of its gathered input row (both store
    paths of the epilogue, whole and ragged column strips)."""
    c = inv.contract(leaves=8, out=out)
    x = synth.randn((T, K), 51).to(DEV)
    W = synth.randn((E, N, K), 52, 0.02).to(DEV)
    ids, _ = inv.moe_route(synth.randn((T, E), 53, dtype=torch.float32).to(DEV), inv.contract(leaves=4))
    offsets, rows, _ = inv.moe_permute(ids, E, inv.contract(leaves=4))
    R = T * 4
    rows = rows.clone()
    rows[5] = T
    rows[R - 1] = -7
    Y = inv.moe_gemm(x, rows, offsets, W, R, c)
    assert torch.isnan(Y[5]).all() and torch.isnan(Y[R - 1]).all()
    offs = offsets.cpu().numpy()
    for e in range(E):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        good = [r for r in range(r0, r1) if r not in (5, R - 1)]
        if not good:
            continue
        gi = torch.as_tensor(good, device=DEV)
        ref = inv.gemm(x[rows[gi].long()].contiguous(), W[e], c)
        assert bitwise_equal(Y[gi], ref), e


def test_grouped_gemm_rows_equal_plain_gemm(inv, moe_full):
    """A grouped row is bitwise what the plain K-leaf GEMM gives for it alone."""
    d = moe_full
    c = inv.contract(leaves=8)
    T = 512
    ids, w = inv.moe_route(d["logits"][:T].contiguous(), c)
    offsets, rows, slot = inv.moe_permute(ids, 128, c)
    GU = inv.moe_gemm(d["x"], rows, offsets, d["W1"], T * 8, c)
    offs = offsets.cpu().numpy()
    for e in (0, 5, 127):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        if r1 == r0:
            continue
        ref = inv.gemm(d["x"][rows[r0:r1].long()].contiguous(), d["W1"][e], c)
        assert bitwise_equal(GU[r0:r1], ref), e


@pytest.mark.parametrize("R,F", [(37, 13), (5, 768), (130, 40)])
def test_swiglu_against_oracle(inv, R, F):
    """Both forms: 16-byte groups (F % 8 == 0) and the scalar form (any F)."""
    gu = synth.randn((R, 2 * F), 31 + F, 2.0)
    a = inv.swiglu(gu.to(DEV), inv.contract())
    check_bf16(a, omoe.swiglu(_np(gu).astype(np.float64)), f"swiglu {R}x{F}")


@pytest.mark.parametrize("T", [1, 3, 1000, 4099])
def test_permute_small_and_ragged(inv, T):
    logits = synth.randn((T, 128), 60 + T, dtype=torch.float32)
    c = inv.contract(leaves=8)
    ids, _ = inv.moe_route(logits.to(DEV), c)
    offsets, rows, slot = inv.moe_permute(ids, 128, c)
    o, r, s = _grouping(ids.cpu().numpy(), 128)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(rows.cpu().numpy(), r)
    assert np.array_equal(slot.cpu().numpy(), s)


@pytest.mark.parametrize("H,offset", [(2048, 0), (2048, 1), (2046, 0), (6, 0)])
def test_combine_vector_and_scalar_paths(inv, H, offset):
    """The combine's float4 path (H % 4 == 0, Y 16-byte aligned) and its
    per-element path (a Y pointer 4 bytes off, or H % 4 != 0) both replay the
    oracle's combine bit for bit."""
    T, KK, rows = 64, 8, 300
    g = torch.Generator().manual_seed(1000 * H + offset)
    flat = torch.randn(rows * H + 4, generator=g).to(DEV)
    Y = flat[offset:offset + rows * H].view(rows, H)
    w = torch.rand((T, KK), generator=g).to(DEV)
    slot = torch.randint(0, rows, (T, KK), generator=g, dtype=torch.int32).to(DEV)
    out = inv.moe_combine(Y, w, slot, inv.contract(leaves=8))
    ref = omoe.combine(Y.cpu().numpy()[slot.cpu().numpy()], w.cpu().numpy())
    assert np.array_equal(_np(out), ref.astype(np.float32))


def test_moe_full_size_sampled_tokens_against_oracle(inv, moe_full):
    """The full 8192-token layer (persistent multi-tile grouped launches, about
    512 grouped rows per expert), checked stage by stage against the oracle on
    16 sampled tokens: every grouped row of their 8 experts (gate/up, SwiGLU,
    down) and their combined outputs, replayed bit for bit."""
    d = moe_full
    c = inv.contract(leaves=8)
    st = {}
    out = inv.moe_layer(d["x"], d["logits"], d["W1"], d["W2"], c, c, out_stage=st)
    toks = np.linspace(0, 8191, 16).astype(int)
    ids = st["ids"].cpu().numpy()
    slot = st["slot"].cpu().numpy()
    rows = st["rows"].cpu().numpy()
    offs = st["offsets"].cpu().numpy()
    oid, ow = omoe.route(d["logits"][toks].double().cpu().numpy(), 8)
    assert np.array_equal(ids[toks], oid)
    assert np.allclose(st["w"][toks].cpu().numpy(), ow, rtol=1e-6, atol=0)
    W1, W2 = _Experts(d["W1"]), _Experts(d["W2"])
    GU, A, Y = st["GU"], st["A"], st["Y"]
    for t in toks:   # each (token, expert) pair sits in its expert's group and gathers its token
        for j in range(8):
            e, r = ids[t, j], slot[t, j]
            assert offs[e] <= r < offs[e + 1] and rows[r] == t
    deep = 0
    for e in np.unique(ids[toks]):
        gr = np.sort(slot[toks][ids[toks] == e])    # grouped rows of the sampled tokens
        deep += int(np.sum(gr - offs[e] >= 128)) if offs[e + 1] - offs[e] >= 500 else 0
        gi = torch.as_tensor(gr, device=DEV)
        xr = _np(d["x"][torch.as_tensor(rows[gr], device=DEV).long()]).astype(np.float64)
        gu = _np(GU[gi])
        check_bf16(gu, omoe.gate_up(xr, W1[e]), f"gate/up e={e}")
        check_bf16(A[gi], omoe.swiglu(gu), f"swiglu e={e}")
        check_fp32_gemm(Y[gi].cpu().numpy(), omoe.down(_np(A[gi]).astype(np.float64), W2[e]), f"down e={e}")
    assert deep >= 16, deep   # rows past the first 128-row tile of well-filled experts were compared
    Yn = Y.cpu().numpy()
    ref = omoe.combine(Yn[slot[toks]], st["w"][toks].cpu().numpy())
    assert np.array_equal(_np(out[toks]), ref.astype(np.float32))
