"""Split-KV attention on the GPU: oracle parity and bitwise invariance.

IsoExec blog, "Unified execution contract": the split-KV partition count is a
pinned contract constant. RL-Kernel write-up, section 4: the attention
softmax over the visible keys is an LSE reduction whose blocks merge by the
two-block rule; section 7: fixed block partition, chunk order and
rescale-merge order. A decode row must equal the same position's prefill row.
"""

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from split_invariant_deterministic_amd import synth
from tests.helpers import bitwise_equal, check_bf16, mismatch_report

pytestmark = pytest.mark.gpu

DEV = "cuda"
EDGE = [1, 2, 15, 16, 17, 63, 64, 65, 1023, 1024, 1025]


@pytest.fixture(scope="module")
def inv():
    from split_invariant_deterministic_amd import inv as m
    return m


def _dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


def _oracle(d, Hkv=8):
    q = d["q"].float().cpu().numpy()
    k = d["k"].float().cpu().numpy()
    v = d["v"].float().cpu().numpy()
    return oatt.attention(q, k, v, d["cu_seqlens"].cpu().numpy(), d["q_seq"].cpu().numpy(),
                          d["q_pos"].cpu().numpy(), Hkv)


def _run(inv, d, c):
    return inv.decode_attn(d["q"], d["k"], d["v"], d["cu_seqlens"], d["q_seq"], d["q_pos"], c)


@pytest.mark.parametrize("kv_chunk,split_kv", [(64, 16), (32, 4), (128, 1), (64, 32)])
def test_edge_lengths_against_oracle(inv, kv_chunk, split_kv):
    d = synth.attn(torch.tensor(EDGE), seed=1)
    out = _run(inv, _dev(d), inv.contract(split_kv=split_kv, kv_chunk=kv_chunk))
    check_bf16(out, _oracle(d), f"edge lengths chunk {kv_chunk} splits {split_kv}")


@pytest.mark.parametrize("Hq,Hkv,kv_chunk,split_kv", [(2, 2, 64, 16), (8, 1, 64, 4), (16, 8, 32, 16),
                                                      (32, 4, 128, 8), (64, 4, 64, 16), (256, 16, 64, 2)])
def test_head_groups_against_oracle(inv, Hq, Hkv, kv_chunk, split_kv):
    # GQA groups of 1 to 16 query heads per kv head (the columns of the score MFMA), 1 to 16 kv
    # heads (the key stride the per-chunk buffer ranges use), every chunk size
    lengths = [1, 17, 64, 65, 300, 1025]
    d = synth.attn(torch.tensor(lengths), Hq=Hq, Hkv=Hkv, seed=7)
    out = _run(inv, _dev(d), inv.contract(split_kv=split_kv, kv_chunk=kv_chunk))
    check_bf16(out, _oracle(d, Hkv), f"Hq {Hq} Hkv {Hkv} chunk {kv_chunk} splits {split_kv}")


def test_full_group_rows_equal_batch(inv):
    # 16 query heads per kv head fill all 16 columns: single rows against the batch, bitwise
    d = _dev(synth.attn(torch.tensor([700, 33, 2049, 64]), Hq=128, Hkv=8, seed=8))
    c = inv.contract()
    full = _run(inv, d, c)
    for i in range(4):
        one = dict(d)
        one["q"] = d["q"][i:i + 1].contiguous()
        one["q_seq"] = d["q_seq"][i:i + 1].contiguous()
        one["q_pos"] = d["q_pos"][i:i + 1].contiguous()
        assert bitwise_equal(_run(inv, one, c), full[i:i + 1]), i


def test_long_context_against_oracle(inv):
    d = synth.attn(torch.tensor([32768, 5000, 2049]), seed=2)
    out = _run(inv, _dev(d), inv.contract())
    check_bf16(out, _oracle(d), "long")


@pytest.mark.parametrize("kv_chunk", [32, 64, 128])
def test_keys_past_the_row_are_never_read(inv, kv_chunk):
    # every K and V row after a query's visible keys holds NaN (inside the same allocation, and
    # past the last sequence); the per-chunk buffer ranges end at each row's last visible key,
    # so the outputs equal those with finite rows, bit for bit (a read of a NaN row would
    # survive the zero probability as NaN)
    lengths = [1, 17, 64, 65, 300, 1025, 2000]
    d = synth.attn(torch.tensor(lengths), seed=10)
    g = torch.Generator().manual_seed(10)
    pos = [int(torch.randint(0, L, (1,), generator=g)) for L in lengths]
    pos[0], pos[-1] = 0, 1000  # a single key, and a row whose chunk ends mid-sequence
    d["q_pos"] = torch.tensor(pos, dtype=torch.int32)
    c = inv.contract(kv_chunk=kv_chunk)
    clean = _run(inv, _dev(d), c)
    T = int(d["cu_seqlens"][-1])
    k = torch.full((T + 256,) + tuple(d["k"].shape[1:]), float("nan"), dtype=torch.bfloat16)
    v = k.clone()
    k[:T], v[:T] = d["k"], d["v"]
    for i, L in enumerate(lengths):
        s0 = int(d["cu_seqlens"][i])
        k[s0 + pos[i] + 1:s0 + L] = float("nan")
        v[s0 + pos[i] + 1:s0 + L] = float("nan")
    dn = _dev(d)
    kd, vd = k.to(DEV), v.to(DEV)
    dn["k"], dn["v"] = kd[:T], vd[:T]
    assert bitwise_equal(_run(inv, dn, c), clean)


def test_single_key_returns_v0_bitwise(inv):
    d = _dev(synth.attn(torch.tensor([1, 1, 1]), seed=3))
    out = _run(inv, d, inv.contract()).cpu()
    v = d["v"].cpu()
    for i in range(3):
        for h in range(32):
            assert torch.equal(out[i, h].view(torch.int16), v[i, h // 4].view(torch.int16))


def _prefill_rows(d, positions):
    """Query rows of sequence 0 at the given positions (q drawn per position)."""
    g = torch.Generator().manual_seed(99)
    L = int(d["cu_seqlens"][1])
    qall = synth.randn((L, 32, 128), 12345)
    pos = torch.as_tensor(positions, dtype=torch.int32)
    return {
        "q": qall[pos.long()].contiguous(),
        "k": d["k"], "v": d["v"], "cu_seqlens": d["cu_seqlens"],
        "q_seq": torch.zeros(len(positions), dtype=torch.int32),
        "q_pos": pos,
    }


def test_decode_equals_prefill_rows(inv):
    L = 3000
    d = synth.attn(torch.tensor([L]), seed=4)
    c = inv.contract()
    positions = list(range(L))
    pre = _dev(_prefill_rows(d, positions))
    full = _run(inv, pre, c)
    # decode: one row at a time (the last row of a shorter context), at sampled positions
    for p in [0, 1, 63, 64, 65, 1023, 1024, 2047, 2998, 2999]:
        one = _dev(_prefill_rows(d, [p]))
        assert bitwise_equal(_run(inv, one, c)[0], full[p]), p
    # and a mixed batch of rows in another order
    sel = [2999, 5, 1500, 64, 0]
    mix = _dev(_prefill_rows(d, sel))
    assert bitwise_equal(_run(inv, mix, c), full[sel])
    rows = [0, 64, 2999]
    sub = _prefill_rows(d, rows)
    check_bf16(full[rows], _oracle(sub), "prefill rows")


@pytest.fixture(scope="module")
def big_batch():
    lengths = synth.attn_lengths(256, 32768, seed=0)
    d = synth.attn(lengths, seed=0, device=DEV)
    d["cu_seqlens"] = d["cu_seqlens"].to(DEV)
    d["q_seq"] = d["q_seq"].to(DEV)
    d["q_pos"] = d["q_pos"].to(DEV)
    return d


def test_batch_invariance_256(inv, big_batch):
    d = big_batch
    c = inv.contract()
    full = _run(inv, d, c)
    for B in (1, 8, 64):
        sub = dict(d)
        sub["q"] = d["q"][:B].contiguous()
        sub["q_seq"] = d["q_seq"][:B].contiguous()
        sub["q_pos"] = d["q_pos"][:B].contiguous()
        n, bad, dmax = mismatch_report(_run(inv, sub, c), full[:B])
        assert bad == 0, f"B={B}: {bad}/{n}, max {dmax}"
    # emulated context-parallel ranks: split ranges computed separately, then one combine
    for R in (2, 4, 16):
        ws = inv.attn_workspace(d["q"], c)
        for r in range(R):
            inv.attn_splits(d["q"], d["k"], d["v"], d["cu_seqlens"], d["q_seq"], d["q_pos"],
                            r * 16 // R, (r + 1) * 16 // R, c, ws)
        assert bitwise_equal(inv.attn_combine(ws, 256, 32, 128, c), full), R
    # sampled rows against the oracle (their own sequences only)
    for i in (0, 17):
        s0, s1 = int(d["cu_seqlens"][i]), int(d["cu_seqlens"][i + 1])
        one = {"q": d["q"][i:i + 1].cpu(), "k": d["k"][s0:s1].cpu(), "v": d["v"][s0:s1].cpu(),
               "cu_seqlens": torch.tensor([0, s1 - s0], dtype=torch.int32),
               "q_seq": torch.zeros(1, dtype=torch.int32), "q_pos": torch.tensor([s1 - s0 - 1], dtype=torch.int32)}
        check_bf16(full[i:i + 1], _oracle(one), f"row {i}")


def test_split_ranges_small_batch(inv, big_batch):
    # 2 to 64 rows are dispatched longest first: split ranges computed separately (emulated
    # context-parallel ranks) still merge to the full launch's bits, at 8 and 64 rows
    d = big_batch
    c = inv.contract()
    for B in (8, 64):
        q = d["q"][:B].contiguous()
        qs, qp = d["q_seq"][:B].contiguous(), d["q_pos"][:B].contiguous()
        full = _run(inv, {"q": q, "k": d["k"], "v": d["v"], "cu_seqlens": d["cu_seqlens"], "q_seq": qs,
                          "q_pos": qp}, c)
        for R in (2, 16):
            ws = inv.attn_workspace(q, c)
            for r in reversed(range(R)):
                inv.attn_splits(q, d["k"], d["v"], d["cu_seqlens"], qs, qp, r * 16 // R, (r + 1) * 16 // R, c, ws)
            assert bitwise_equal(inv.attn_combine(ws, B, 32, 128, c), full), (B, R)


def test_left_fold_changes_bits(inv, big_batch):
    d = big_batch
    bal = _run(inv, d, inv.contract())
    fold = _run(inv, d, inv.contract(tree="left_fold"))
    _, bad, _ = mismatch_report(bal, fold)
    assert bad > 0


def test_bad_positions_give_nan(inv):
    d = _dev(synth.attn(torch.tensor([10, 20]), seed=5))
    d["q_pos"] = torch.tensor([10, 19], dtype=torch.int32, device=DEV)  # row 0: past its sequence
    out = _run(inv, d, inv.contract()).cpu()
    assert torch.isnan(out[0].float()).all() and not torch.isnan(out[1].float()).any()
    d["q_seq"] = torch.tensor([2, 1], dtype=torch.int32, device=DEV)    # row 0: no such sequence
    d["q_pos"] = torch.tensor([0, 19], dtype=torch.int32, device=DEV)
    out = _run(inv, d, inv.contract()).cpu()
    assert torch.isnan(out[0].float()).all() and not torch.isnan(out[1].float()).any()


def test_repeat_runs(inv):
    d = _dev(synth.attn(torch.tensor(EDGE), seed=6))
    c = inv.contract()
    first = _run(inv, d, c)
    for _ in range(20):
        assert bitwise_equal(_run(inv, d, c), first)
