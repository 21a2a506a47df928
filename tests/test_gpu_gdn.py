"""Gated DeltaNet under the CPR schedule on the GPU: prefill = decode bit for
bit, batch invariance, oracle parity.

IsoExec blog, "Chunkwise-parallel recurrent (CPR) GDN": boundary states by a
first pass, outputs by the recurrence from each chunk's boundary, decode
resynchronised at every boundary, so prefill, training forward and decode
share one rounding schedule. The oracle (float64) runs the same schedule and
equals the plain recurrence up to float64 rounding.
"""

import numpy as np
import pytest
import torch

from oracle import gdn as ogdn
from split_invariant_deterministic_amd import synth
from tests.helpers import bitwise_equal, mismatch_report

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def inv():
    from split_invariant_deterministic_amd import inv as m
    return m


def _dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


def _np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _oracle(d, C):
    return ogdn.gdn_layer(_np64(d["q"]), _np64(d["k"]), _np64(d["v"]), _np64(d["g"]), _np64(d["beta"]),
                          d["cu_seqlens"].cpu().numpy(), C)


def check_gdn(gpu, ora, what):
    """|gpu - ora| <= 1e-4 * rms(ora) + 1e-4 * |ora| elementwise (fp32 chains over a chunk and
    the boundary updates; a wrong term or index moves outputs by O(rms))."""
    g = gpu.float().cpu().numpy().astype(np.float64)
    rms = float(np.sqrt(np.mean(ora * ora)))
    lim = 1e-4 * rms + 1e-4 * np.abs(ora)
    bad = np.abs(g - ora) > lim
    assert not bad.any(), f"{what}: {int(bad.sum())} outside, max err {np.abs(g - ora).max():.3g} rms {rms:.3g}"


@pytest.mark.parametrize("C", [32, 64])
def test_prefill_against_oracle(inv, C):
    d = synth.gdn([1, 70, 130, 64], H=2, seed=1)
    c = inv.contract(kv_chunk=C, out="fp32")
    dd = _dev(d)
    out = inv.gdn_prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["cu_seqlens"], c)
    check_gdn(out, _oracle(d, C), f"C={C}")
    # the bf16 boundary is the RNE of the fp32 result
    ob = inv.gdn_prefill(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["cu_seqlens"],
                         inv.contract(kv_chunk=C, out="bf16"))
    assert bitwise_equal(ob, out.to(torch.bfloat16))


@pytest.mark.parametrize("C", [32, 64])
def test_prefill_then_decode_is_bitwise_one_prefill(inv, C):
    lengths = [150, 150]
    d = _dev(synth.gdn(lengths, H=3, seed=2))
    c = inv.contract(kv_chunk=C, out="fp32")
    full = inv.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], c)
    H = 3
    for L0 in (0, 1, C - 1, C, C + 1, 2 * C, 100):
        # prefill both sequences to L0 tokens, then decode one token at a time
        cache = inv.gdn_cache(c, 2, H, DEV)
        idx = torch.cat([torch.arange(0, L0), torch.arange(150, 150 + L0)]).to(DEV)
        cu0 = torch.tensor([0, L0, 2 * L0], dtype=torch.int32, device=DEV)
        if L0 > 0:
            inv.gdn_prefill(d["q"][idx].contiguous(), d["k"][idx].contiguous(), d["v"][idx].contiguous(),
                            d["g"][idx].contiguous(), d["beta"][idx].contiguous(), cu0, c, cache=cache)
        for p in range(L0, 150):
            rows = torch.tensor([p, 150 + p], device=DEV)
            pos = torch.full((2,), p, dtype=torch.int32, device=DEV)
            o = inv.gdn_decode(d["q"][rows].contiguous(), d["k"][rows].contiguous(), d["v"][rows].contiguous(),
                               d["g"][rows].contiguous(), d["beta"][rows].contiguous(), pos, cache, c)
            n, bad, dmax = mismatch_report(o, full[rows])
            assert bad == 0, f"C={C} L0={L0} token {p}: {bad}/{n} differ, max {dmax}"


def test_decode_positions_may_differ_across_the_batch(inv):
    C = 32
    d = _dev(synth.gdn([90, 90], H=2, seed=3))
    c = inv.contract(kv_chunk=C, out="fp32")
    full = inv.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], c)
    cache = inv.gdn_cache(c, 2, 2, DEV)
    # sequence 0 prefilled to 31 tokens, sequence 1 to 40, then decoded side by side
    idx = torch.cat([torch.arange(0, 31), torch.arange(90, 130)]).to(DEV)
    cu0 = torch.tensor([0, 31, 71], dtype=torch.int32, device=DEV)
    inv.gdn_prefill(d["q"][idx].contiguous(), d["k"][idx].contiguous(), d["v"][idx].contiguous(),
                    d["g"][idx].contiguous(), d["beta"][idx].contiguous(), cu0, c, cache=cache)
    for step in range(45):
        p0, p1 = 31 + step, 40 + step
        rows = torch.tensor([p0, 90 + p1], device=DEV)
        pos = torch.tensor([p0, p1], dtype=torch.int32, device=DEV)
        o = inv.gdn_decode(d["q"][rows].contiguous(), d["k"][rows].contiguous(), d["v"][rows].contiguous(),
                           d["g"][rows].contiguous(), d["beta"][rows].contiguous(), pos, cache, c)
        assert bitwise_equal(o, full[rows]), step


def test_batch_composition_invariance(inv):
    C = 64
    lengths = [200, 7, 129, 64]
    d = _dev(synth.gdn(lengths, H=2, seed=4))
    c = inv.contract(kv_chunk=C, out="fp32")
    full = inv.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], c)
    cu = d["cu_seqlens"].tolist()
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        one = inv.gdn_prefill(d["q"][a:b].contiguous(), d["k"][a:b].contiguous(), d["v"][a:b].contiguous(),
                              d["g"][a:b].contiguous(), d["beta"][a:b].contiguous(),
                              torch.tensor([0, b - a], dtype=torch.int32, device=DEV), c)
        assert bitwise_equal(one, full[a:b]), s


def test_no_writes_keep_the_state_zero(inv):
    """beta = 0: nothing is written, every output is exactly zero (decode too)."""
    d = _dev(synth.gdn([100], H=2, seed=5))
    d["beta"] = torch.zeros_like(d["beta"])
    c = inv.contract(kv_chunk=32, out="fp32")
    out = inv.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], c)
    assert torch.count_nonzero(out).item() == 0


def test_bad_decode_position_is_nan(inv):
    d = _dev(synth.gdn([2, 2], H=2, seed=6))
    c = inv.contract(kv_chunk=32, out="fp32")
    cache = inv.gdn_cache(c, 2, 2, DEV)
    snap = cache.clone()
    pos = torch.tensor([-1, 0], dtype=torch.int32, device=DEV)
    rows = torch.tensor([0, 2], device=DEV)
    o = inv.gdn_decode(d["q"][rows].contiguous(), d["k"][rows].contiguous(), d["v"][rows].contiguous(),
                       d["g"][rows].contiguous(), d["beta"][rows].contiguous(), pos, cache, c)
    assert torch.isnan(o[0]).all() and not torch.isnan(o[1]).any()
    per = cache.numel() // 2
    assert torch.equal(cache[:per], snap[:per])  # the bad sequence's cache is untouched


def test_workload_shape_decode_tail_and_sampled_oracle(inv):
    """5 sequences of 2048 tokens, 16 heads: the last 70 tokens decoded after a prefill of
    1978 equal the full prefill bit for bit; two (sequence, head) pairs against the oracle."""
    C = 64
    d = synth.gdn([2048] * 5, H=16, seed=0, device=DEV)
    c = inv.contract(kv_chunk=C, out="fp32")
    full = inv.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], c)
    cache = inv.gdn_cache(c, 5, 16, DEV)
    L0 = 1978
    idx = torch.cat([torch.arange(s * 2048, s * 2048 + L0) for s in range(5)]).to(DEV)
    cu0 = torch.arange(0, 6, dtype=torch.int32, device=DEV) * L0
    inv.gdn_prefill(d["q"][idx].contiguous(), d["k"][idx].contiguous(), d["v"][idx].contiguous(),
                    d["g"][idx].contiguous(), d["beta"][idx].contiguous(), cu0, c, cache=cache)
    for p in range(L0, 2048):
        rows = (torch.arange(5, device=DEV) * 2048 + p)
        pos = torch.full((5,), p, dtype=torch.int32, device=DEV)
        o = inv.gdn_decode(d["q"][rows].contiguous(), d["k"][rows].contiguous(), d["v"][rows].contiguous(),
                           d["g"][rows].contiguous(), d["beta"][rows].contiguous(), pos, cache, c)
        assert bitwise_equal(o, full[rows]), p
    for s, h in ((0, 0), (4, 15)):
        sl = slice(s * 2048, (s + 1) * 2048)
        qh, kh, alpha = ogdn.prep(_np64(d["q"][sl, h]), _np64(d["k"][sl, h]), _np64(d["g"][sl, h]))
        o, _, _ = ogdn.cpr(qh, kh, _np64(d["v"][sl, h]), alpha, _np64(d["beta"][sl, h]), C)
        check_gdn(full[sl, h], o, f"seq {s} head {h}")


def test_chunk_size_moves_bits(inv):
    """Teeth: the boundary placement is part of the rounding schedule, so C = 32 and C = 64
    differ in some bits (both within the oracle bar)."""
    d = _dev(synth.gdn([300], H=2, seed=7))
    o32 = inv.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], inv.contract(kv_chunk=32, out="fp32"))
    o64 = inv.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], inv.contract(kv_chunk=64, out="fp32"))
    n, bad, dmax = mismatch_report(o32, o64)
    assert bad > 0
    assert bitwise_equal(o32[:32], o64[:32])  # before the first boundary both run the same recurrence
