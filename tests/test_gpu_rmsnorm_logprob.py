"""RMSNorm and selected-token logprob on the GPU: oracle parity, closed forms
and bitwise invariance.

RL-Kernel write-up, section 4: RMSNorm is the reduction class over the
hidden dimension; LSE = m + log sum exp(x - m); a token's logprob is its
logit minus the LSE over the whole vocabulary; vocabulary blocks merge as
m = max(m1, m2), s = s1 e^(m1-m) + s2 e^(m2-m) in a pinned order. Section 7:
per-shard statistics merged in a fixed vocabulary-tile order.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import logprob as olp
from oracle import rmsnorm as orms
from split_invariant_deterministic_amd import synth
from tests.helpers import bitwise_equal, check_bf16, check_logprob, mismatch_report

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DEV = "cuda"


@pytest.fixture(scope="module")
def inv():
    from split_invariant_deterministic_amd import inv as m
    return m


def _np(t):
    return t.float().cpu().numpy()


# ------------------------------------------------------------------ RMSNorm

@pytest.mark.parametrize("M,H", [(8, 256), (37, 4096), (5, 8), (3, 1000), (2, 16384), (300, 512)])
def test_rmsnorm_against_oracle(inv, M, H):
    d = synth.rmsnorm(M, H, seed=H)
    y = inv.rmsnorm(d["x"].to(DEV), d["gamma"].to(DEV), inv.contract())
    check_bf16(y, orms.rmsnorm(_np(d["x"]), _np(d["gamma"]), 1e-6), f"rmsnorm {M}x{H}")


def test_rmsnorm_tiny_config(inv):
    t = synth.tiny(0)
    y = inv.rmsnorm(t["x"].to(DEV), t["gamma"].to(DEV), inv.contract(eps=1e-6))
    check_bf16(y, orms.rmsnorm(_np(t["x"]), _np(t["gamma"]), 1e-6), "tiny")


def test_rmsnorm_closed_forms(inv):
    H = 256
    x = torch.zeros((3, H), dtype=torch.bfloat16)
    x[1] = 1.0
    x[2, 17] = 1.0
    y = inv.rmsnorm(x.to(DEV), torch.ones(H, dtype=torch.bfloat16, device=DEV), inv.contract()).cpu()
    assert torch.all(y[0] == 0)
    assert torch.all(y[1] == 1.0)
    assert y[2, 17].item() == 16.0 and int((y[2] != 0).sum()) == 1


def test_rmsnorm_batch_invariance(inv):
    d = synth.rmsnorm(4096, 4096, seed=0, device=DEV)
    c = inv.contract()
    full = inv.rmsnorm(d["x"], d["gamma"], c)
    for M in (1, 7, 64, 512):
        assert bitwise_equal(inv.rmsnorm(d["x"][:M].contiguous(), d["gamma"], c), full[:M]), M
    perm = torch.randperm(4096, generator=torch.Generator().manual_seed(1)).to(DEV)
    assert bitwise_equal(inv.rmsnorm(d["x"][perm].contiguous(), d["gamma"], c), full[perm])
    rows = torch.tensor([0, 1, 511, 4095])
    check_bf16(full[rows.to(DEV)], orms.rmsnorm(_np(d["x"][rows.to(DEV)]), _np(d["gamma"]), 1e-6), "sampled")


# ------------------------------------------------------------------ logprob

def _rand_logits(M, V, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((M, V), generator=g) * scale


@pytest.mark.parametrize("M,V,C", [(8, 512, 4), (5, 151936, 64), (9, 1000, 8), (4, 64, 64), (3, 7, 1),
                                   (6, 2374 * 64 + 37, 64), (2, 40000, 512), (3, 10000, 2)])
def test_logprob_against_oracle(inv, M, V, C):
    x = _rand_logits(M, V, V)
    t = torch.randint(0, V, (M,), generator=torch.Generator().manual_seed(C)).to(torch.int32)
    lp = inv.logprob(x.to(DEV), t.to(DEV), inv.contract(leaves=C))
    xd = x.double().numpy()
    check_logprob(lp, olp.logprob(xd, t.numpy()), f"{M}x{V}/{C}", lse=olp.lse(xd))


def test_logprob_peaked_logits(inv):
    """Trained-model-like peaked rows (logits x 10): reported, same bar."""
    x = _rand_logits(16, 151936, 11, scale=10.0)
    t = torch.argmax(x, 1).to(torch.int32)
    t[::2] = torch.randint(0, 151936, (8,), generator=torch.Generator().manual_seed(2)).to(torch.int32)
    lp = inv.logprob(x.to(DEV), t.to(DEV), inv.contract(leaves=64))
    xd = x.double().numpy()
    check_logprob(lp, olp.logprob(xd, t.numpy()), "peaked", lse=olp.lse(xd))


def test_logprob_constant_logits(inv):
    g = json.load(open(os.path.join(GOLDEN, "logprob_constant.json")))
    V = g["V"]
    x = torch.full((3, V), g["value"], dtype=torch.float32, device=DEV)
    t = torch.tensor([0, 5, V - 1], dtype=torch.int32, device=DEV)
    c = inv.contract(leaves=g["chunks"])
    lp = inv.logprob(x, t, c)
    assert np.allclose(lp.cpu().numpy(), g["expected"], rtol=1e-6, atol=0)
    stats, _ = inv.logprob_partials(x, t, 0, g["chunks"], c)
    assert torch.all(stats[:, :, 1] == g["chunk_sum"])  # exp2(0) = 1 summed exactly


def test_logprob_bad_targets_are_nan(inv):
    x = _rand_logits(4, 300, 1).to(DEV)
    t = torch.tensor([-1, 300, 5, 1 << 30], dtype=torch.int32, device=DEV)
    lp = inv.logprob(x, t, inv.contract(leaves=4)).cpu()
    assert torch.isnan(lp[0]) and torch.isnan(lp[1]) and torch.isnan(lp[3]) and not torch.isnan(lp[2])


def test_logprob_strided_rows(inv):
    big = _rand_logits(6, 1200, 4).to(DEV)
    x = big[:, :1000]
    t = torch.arange(6, dtype=torch.int32, device=DEV) * 150
    c = inv.contract(leaves=8)
    assert bitwise_equal(inv.logprob(x, t, c), inv.logprob(x.contiguous(), t, c))


@pytest.fixture(scope="module")
def lm_logits():
    g = torch.Generator(device=DEV).manual_seed(77)
    x = torch.randn((4096, 151936), generator=g, device=DEV) * 1.3
    t = torch.randint(0, 151936, (4096,), generator=g, device=DEV).to(torch.int32)
    return x, t


def test_logprob_batch_invariance_lm_head_size(inv, lm_logits):
    x, t = lm_logits
    c = inv.contract(leaves=64)
    full = inv.logprob(x, t, c)
    for M in (1, 7, 64, 512):
        assert bitwise_equal(inv.logprob(x[:M], t[:M], c), full[:M]), M
    one = torch.stack([inv.logprob(x[i:i + 1], t[i:i + 1], c)[0] for i in (0, 1000, 4095)])
    assert bitwise_equal(one, full[[0, 1000, 4095]])
    rows = [0, 1, 2047, 4095]
    xr = x[rows].double().cpu().numpy()
    check_logprob(full[rows], olp.logprob(xr, t[rows].cpu().numpy()), "sampled", lse=olp.lse(xr))


def test_logprob_vocab_shards_are_bitwise_equal(inv, lm_logits):
    x, t = lm_logits
    x, t = x[:256], t[:256]
    c = inv.contract(leaves=64)
    base = inv.logprob(x, t, c)
    for R in (1, 2, 4, 8):
        stats = torch.full((256, 64, 2), float("nan"), device=DEV)
        tl = torch.full((256,), float("nan"), device=DEV)
        for r in range(R):
            inv.logprob_partials(x, t, r * 64 // R, (r + 1) * 64 // R, c, stats, tl)
        assert bitwise_equal(inv.logprob_combine(stats, tl, t, x.shape[1], c), base), R


def test_logprob_left_fold_changes_bits(inv, lm_logits):
    x, t = lm_logits
    bal = inv.logprob(x[:1024], t[:1024], inv.contract(leaves=64))
    fold = inv.logprob(x[:1024], t[:1024], inv.contract(leaves=64, tree="left_fold"))
    _, bad, dmax = mismatch_report(bal, fold)
    assert bad > 0 and dmax < 1e-4


def test_logprob_chunk_stats_against_oracle(inv):
    x = _rand_logits(3, 9000, 5)
    t = torch.zeros(3, dtype=torch.int32)
    stats, _ = inv.logprob_partials(x.to(DEV), t.to(DEV), 0, 16, inv.contract(leaves=16))
    ms, ss = olp.chunk_stats(x.double().numpy(), 16)
    s = stats.cpu().numpy()
    assert np.array_equal(s[:, :, 0], ms.astype(np.float32))          # the max is exact
    assert np.allclose(s[:, :, 1], ss, rtol=5e-6, atol=0)   # fp32 exp2 + lane sums


def test_logprob_sum_to_one(inv):
    """Every token's probability from the kernel sums to one over the vocabulary."""
    V = 3000
    x = _rand_logits(2, V, 8, 2.0).to(DEV)
    c = inv.contract(leaves=8)
    tot = []
    for r in range(2):
        xs = x[r:r + 1].expand(V, V).contiguous()
        lp = inv.logprob(xs, torch.arange(V, dtype=torch.int32, device=DEV), c)
        tot.append(math.fsum(np.exp(lp.double().cpu().numpy())))
    assert np.allclose(tot, 1.0, rtol=0, atol=2e-5)


@pytest.mark.parametrize("V,C", [(9000, 16), (151936, 64), (3000, 1)])
def test_logprob_masked_chunks(inv, V, C):
    """-inf logits (a masked vocabulary range): a fully masked chunk is the
    merge identity (-inf, 0) and scattered -inf entries add nothing, so the
    result stays finite and within the bar of the oracle's plain definition;
    the 16-column block schedule agrees within the same bar."""
    x = _rand_logits(4, V, 12)
    if C > 1:
        a, e = olp.chunk_bounds(V, C)[1]
        x[0, a:e] = float("-inf")                                # chunk 1 fully masked
    x[1, ::7] = float("-inf")                                    # scattered
    x[2, : (V // 2)] = float("-inf")                             # the first half of the row
    x[3, -17:] = float("-inf")                                   # a ragged tail
    t = torch.tensor([3, 5, V - 1, 0], dtype=torch.int32)
    xd = x.double().numpy()
    ora = olp.logprob(xd, t.numpy())
    assert np.all(np.isfinite(ora))
    c = inv.contract(leaves=C)
    lp = inv.logprob(x.to(DEV), t.to(DEV), c)
    check_logprob(lp, ora, f"masked {V}/{C}", lse=olp.lse(xd))
    if C > 1:
        stats, _ = inv.logprob_partials(x.to(DEV), t.to(DEV), 0, C, c)
        s = stats.cpu()
        assert s[0, 1, 0].item() == float("-inf") and s[0, 1, 1].item() == 0.0
    lb = inv.logprob_block16(x.to(DEV), t.to(DEV), inv.contract(out="fp32"))
    check_logprob(lb, ora, f"masked block16 {V}", lse=olp.lse(xd))
