"""Fused LM head + selected-token logprob on the GPU: oracle parity, bitwise
equality with the unfused path, and batch invariance.

RL-Kernel write-up, section 4: lp = x[t] - LSE over the vocabulary, with
vocabulary blocks carrying (m, s) statistics merged in a fixed order;
section 7: logits stay fp32. The fused kernel reduces 16-column blocks (one
MFMA output block) in the GEMM epilogue and never stores the logits; the
unfused twin (inv_logprob_block16 on inv_gemm's fp32 logits) must give the
same bits, and so must every batch size.
"""

import numpy as np
import pytest
import torch

from oracle import gemm as ogemm
from oracle import logprob as olp
from split_invariant_deterministic_amd import synth
from tests.helpers import bitwise_equal, check_logprob, mismatch_report

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def inv():
    from split_invariant_deterministic_amd import inv as m
    return m


def _np64(t):
    return t.float().cpu().numpy().astype(np.float64)


def test_tiny_against_oracle(inv):
    t = synth.tiny(0)
    h, W, tg = t["x"].to(DEV), t["W"].to(DEV), t["targets"].to(DEV)
    lp = inv.lmhead_logprob(h, W, tg, inv.contract(leaves=4, out="fp32"))
    logits = ogemm.gemm_tree(_np64(t["x"]), _np64(t["W"]), 4, "fp32").astype(np.float64)
    tn = t["targets"].numpy()
    check_logprob(lp, olp.logprob(logits, tn), "tiny", lse=olp.lse(logits))
    check_logprob(lp, olp.logprob_blocks(logits, tn), "tiny blocks", lse=olp.lse(logits))


CASES = [  # M, V, K, leaves: stream kernel (M <= 64) and ring kernel, ragged last block
    (1, 517, 256, 4), (7, 1000, 512, 8), (16, 16, 64, 1), (64, 4099, 256, 8),
    (65, 1000, 256, 2), (130, 2003, 512, 8), (300, 129, 1024, 4),
]


@pytest.mark.parametrize("M,V,K,L", CASES)
def test_fused_equals_unfused_and_oracle(inv, M, V, K, L):
    h = synth.randn((M, K), 300 + M, device="cpu")
    W = synth.randn((V, K), 301 + V, 0.05, device="cpu")
    t = synth.randint(0, V, (M,), 302 + M)
    t[0] = V - 1                       # the ragged last block
    if M > 2:
        t[1] = 0
    hd, Wd, td = h.to(DEV), W.to(DEV), t.to(DEV)
    c = inv.contract(leaves=L, out="fp32")
    ws_f = inv.block16_workspace(M, V, DEV)
    lp_f = inv.lmhead_logprob(hd, Wd, td, c, ws=ws_f)
    logits = inv.gemm(hd, Wd, c)
    ws_u = inv.block16_workspace(M, V, DEV)
    lp_u = inv.logprob_block16(logits, td, c, ws=ws_u)
    assert bitwise_equal(lp_f, lp_u)
    st_f, tl_f = inv.block16_views(ws_f, M, V)
    st_u, tl_u = inv.block16_views(ws_u, M, V)
    assert bitwise_equal(st_f, st_u) and bitwise_equal(tl_f, tl_u)
    # block maxima are exact; the target logit is the logit
    nb = (V + 15) // 16
    padded = torch.full((M, nb * 16), float("-inf"), device=DEV)
    padded[:, :V] = logits
    assert torch.equal(st_f[:, :, 0], padded.view(M, nb, 16).amax(dim=2))
    assert torch.equal(tl_f, logits[torch.arange(M, device=DEV), td.long()])
    # oracle: its own fp32 logits, then the plain definition and the block schedule
    ora_logits = ogemm.gemm_tree(_np64(h), _np64(W), L, "fp32").astype(np.float64)
    tn = t.numpy()
    check_logprob(lp_f, olp.logprob(ora_logits, tn), f"{M}x{V}", lse=olp.lse(ora_logits))
    ms, ss = olp.block_stats(ora_logits)
    assert np.allclose(st_f[:, :, 1].cpu().numpy(), ss, rtol=2e-5, atol=0)


def test_bad_targets_are_nan(inv):
    M, V, K = 6, 300, 256
    h = synth.randn((M, K), 40).to(DEV)
    W = synth.randn((V, K), 41, 0.05).to(DEV)
    t = torch.tensor([-1, V, 0, V - 1, 5, 1 << 30], dtype=torch.int32, device=DEV)
    lp = inv.lmhead_logprob(h, W, t, inv.contract(leaves=8, out="fp32")).cpu()
    assert torch.isnan(lp[[0, 1, 5]]).all() and not torch.isnan(lp[[2, 3, 4]]).any()


def test_probabilities_sum_to_one(inv):
    """Every vocabulary entry's probability through the fused path sums to one."""
    import math
    V, K = 2000, 256
    h = synth.randn((1, K), 50, 2.0).to(DEV)
    W = synth.randn((V, K), 51, 0.1).to(DEV)
    hs = h.expand(V, K).contiguous()
    lp = inv.lmhead_logprob(hs, W, torch.arange(V, dtype=torch.int32, device=DEV),
                            inv.contract(leaves=8, out="fp32"))
    assert abs(math.fsum(np.exp(lp.double().cpu().numpy())) - 1.0) < 2e-5
    assert torch.unique(lp.view(torch.int32)).numel() > 1  # not a degenerate case


@pytest.fixture(scope="module")
def lm():
    return synth.lmhead(M=4096, H=4096, V=151936, seed=0, device=DEV)


def test_lm_head_size_fused_unfused_batch_invariance(inv, lm):
    h, W, t = lm["h"], lm["W"], lm["targets"]
    V = W.shape[0]
    c = inv.contract(leaves=8, out="fp32")
    full = inv.lmhead_logprob(h, W, t, c)
    for M in (1, 7, 64, 65, 512):
        assert bitwise_equal(inv.lmhead_logprob(h[:M].contiguous(), W, t[:M].contiguous(), c), full[:M]), M
    one = torch.stack([inv.lmhead_logprob(h[i:i + 1].contiguous(), W, t[i:i + 1].contiguous(), c)[0]
                       for i in (0, 2047, 4095)])
    assert bitwise_equal(one, full[[0, 2047, 4095]])
    # the unfused twin on the full batch's stored logits
    logits = inv.gemm(h, W, c)
    assert bitwise_equal(inv.logprob_block16(logits, t, c), full)
    # the C-chunk schedule is another contract: close, not bitwise
    other = inv.logprob(logits, t, inv.contract(leaves=64))
    n, bad, dmax = mismatch_report(full, other)
    assert dmax < 1e-4, dmax
    del logits
    # sampled rows against the oracle from the synthetic inputs
    rows = [0, 1, 2047, 4095]
    hs = _np64(h[rows])
    parts = []
    for v0 in range(0, V, 16384):
        parts.append(ogemm.gemm_tree(hs, _np64(W[v0:v0 + 16384]), 8, "fp32").astype(np.float64))
    ora = np.concatenate(parts, axis=1)
    tn = t[rows].cpu().numpy()
    check_logprob(full[rows], olp.logprob(ora, tn), "lm head sampled", lse=olp.lse(ora))


def test_block_merge_left_fold_changes_bits(inv, lm):
    h, W, t = lm["h"][:256].contiguous(), lm["W"], lm["targets"][:256].contiguous()
    logits = inv.gemm(h, W, inv.contract(leaves=8, out="fp32"))
    bal = inv.logprob_block16(logits, t, inv.contract(leaves=8))
    fold = inv.logprob_block16(logits, t, inv.contract(leaves=8, tree="left_fold"))
    _, bad, dmax = mismatch_report(bal, fold)
    assert bad > 0 and dmax < 1e-4


def test_unfused_lm_head_chain_batch_invariance_full_size(inv, lm):
    """The unfused chain at the full LM-head shape (inv_gemm 4096x151936x4096
    with fp32 logits, then the 64-chunk inv_logprob): batch 1 and the prefixes
    give, bit for bit, the rows of batch 4096 -- logits and logprobs."""
    h, W, t = lm["h"], lm["W"], lm["targets"]
    c = inv.contract(leaves=8, out="fp32")
    c64 = inv.contract(leaves=64)
    logits = inv.gemm(h, W, c)
    full = inv.logprob(logits, t, c64)
    for i in (0, 1, 2047, 4095):
        l1 = inv.gemm(h[i:i + 1].contiguous(), W, c)
        assert bitwise_equal(l1[0], logits[i]), i
        assert bitwise_equal(inv.logprob(l1, t[i:i + 1].contiguous(), c64)[0], full[i]), i
    for M in (7, 64, 512):
        lm_ = inv.gemm(h[:M].contiguous(), W, c)
        assert bitwise_equal(lm_, logits[:M]), M
        assert bitwise_equal(inv.logprob(lm_, t[:M].contiguous(), c64), full[:M]), M
        del lm_
    del logits
