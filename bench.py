"""Benchmark of the invariant logprob forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch of seeded
synthetic input, every stage in the library's HIP kernels:

  dense   RMSNorm [4096 x 4096] -> invariant GEMM 4096->12288 -> invariant
          GEMM 12288->4096 (M = 4096 tokens, 8 K-leaves, bf16 out)
  norm    RMSNorm at its bandwidth shape, [65536 x 4096] bf16 (1.07 GB moved)
  attn    split-KV decode attention, 256 sequences with lengths uniform in
          [1, 32768], 32 query / 8 KV heads, head dim 128, 16 splits
  moe     8192 tokens, hidden 2048, 128 experts, top-8, expert FFN
          2048->768->2048 with 8 K-leaves, fixed expert-order combine
  lmhead  RMSNorm -> invariant GEMM 4096->151936 (fp32 logits) -> 64-chunk
          selected-token logprob, 4096 tokens; the fused LM head (logprob
          from 16-column blocks in the GEMM epilogue, no stored logits) is
          timed beside the step, not inside it
  sweep   outside the step, median of 20 launches each: the dense pair at
          M = 1, 7, 64, 512 (prefixes; warm, and rotated over three weight
          copies so the 201 MB never sits in the 256 MB Infinity Cache), next
          to hipBLASLt and the 1-leaf kernel; RMSNorm latency at M = 1 ..
          4096; attention at B = 1, 8, 64 (prefixes of the 256 sequences);
          the MoE layer run as 4 and 16 contiguous token splits; the LM head +
          logprob at M = 1 and 64 (fused, unfused and the fast path); a 1 GiB copy

After the timed steps (never inside them): an ``invariance`` report, GPU
against GPU and counted element by element -- batch size (prefixes and
single rows against the 4096-token batch), emulated rank partitions of the
GEMM leaves and of the key splits, prefill against decode (attention and
Gated DeltaNet), MoE token splits, and 20 more whole steps against the last
timed one; a ``device`` record (CU count, clocks, and the MFMA ceiling: a
register-only loop of the path's MFMA instruction with the shader clock it
held); and ``cpu_oracle_configs``, the oracle timed per configuration on
bounded samples beside ``cpu_baseline``.

Inputs are resident in HBM before the timed region. ``value`` is the
invariant GEMM throughput of the dense stage (its FLOPs over the time of its
two GEMM launches, HIP events on the launch stream); the logprob tokens/s,
per-stage times and the overhead against a non-invariant fast path
(hipBLASLt matmul, torch rms_norm, log_softmax + gather, split count chosen
for occupancy) are reported in the same JSON line, together with the
roofline of the dominant kernel and the CPU oracle timed on a bounded sample.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector, published (packed fp32; without packed ops, which
                            # this library never emits, the ceiling is 78.6)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--invariance-repeats", type=int, default=20,
                   help="whole steps repeated after the timed ones and compared bitwise with the last "
                        "(-1 skips the invariance report)")
    p.add_argument("--stages", default="dense,norm,attn,moe,lmhead,gdn,sweep",
                   help="comma list of dense,norm,attn,moe,lmhead,gdn,sweep (all by default); "
                        "'copy' adds a plain 1 GiB device copy used only to calibrate traffic counters")
    return p.parse_args()


class Timer:
    """Per-stage HIP event pairs on the current stream (where the library launches)."""

    def __init__(self, torch):
        self.torch = torch
        self.ev = {}

    def start(self, name):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        self.ev.setdefault(name, []).append((e0, e1))

    def stop(self, name):
        self.ev[name][-1][1].record()

    def mean_ms(self, name):
        pairs = self.ev.get(name, [])
        return sum(a.elapsed_time(b) for a, b in pairs) / max(len(pairs), 1)

    def reset(self):
        self.ev = {}


_SLEEP = {"cycles": 0}


def median_us(torch, fn, iters=20, warm=5):
    """Median GPU time of one call of ``fn`` over ``iters`` back-to-back calls,
    after ``warm`` untimed ones. A spin kernel keeps the GPU busy while the host
    enqueues the calls, and an event sits between every two calls, so host-side
    marshalling (several µs per call) never shows up as GPU time; the spin is
    lengthened until the host has finished enqueueing before it ends."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    if not _SLEEP["cycles"]:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(1 << 20)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP["cycles"] = int((1 << 20) * 2000.0 / max(e0.elapsed_time(e1) * 1e3, 1.0))  # about 2 ms
    for _ in range(4):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        e_s = torch.cuda.Event(enable_timing=True)
        e_s.record()
        torch.cuda._sleep(_SLEEP["cycles"])
        h0 = time.perf_counter()
        ev[0].record()
        for i in range(iters):
            fn()
            ev[i + 1].record()
        host_us = (time.perf_counter() - h0) * 1e6
        torch.cuda.synchronize()
        if host_us < 0.8 * e_s.elapsed_time(ev[0]) * 1e3:
            break
        _SLEEP["cycles"] *= 2  # the host was still enqueueing when the spin ended: spin longer
    t = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(iters))
    return t[len(t) // 2]


def sweep(torch, inv, synth, X, W_up, W_down, gamma, att, moe, lm, c8, cn, ca, dev):
    """The shape lists of the measurement plan, each kernel at its own roofline."""
    import torch.nn.functional as F
    out = {}
    Hd, Ff = W_up.shape[1], W_up.shape[0]
    # dense pair at small M: HBM-bound on the 201 MB of weights up to M = 64
    sets = [(W_up, W_down), (W_up.clone(), W_down.clone()), (W_up.clone(), W_down.clone())]
    dn = {}
    for M in (1, 7, 64, 512):
        x = X[:M]
        a = torch.empty((M, Ff), dtype=torch.bfloat16, device=dev)
        b = torch.empty((M, Hd), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(inv.workspace_bytes(c8, inv.OP_GEMM, M, Ff, Hd),
                             inv.workspace_bytes(c8, inv.OP_GEMM, M, Hd, Ff), 1), dtype=torch.uint8, device=dev)
        rot = [0]

        def inv_pair(i=None, c=c8):
            wu, wd = sets[rot[0] % 3] if i is None else sets[i]
            rot[0] += 1
            inv.gemm(x, wu, c, out=a, ws=ws)
            inv.gemm(a, wd, c, out=b, ws=ws)

        def fast_pair(i=None):
            wu, wd = sets[rot[0] % 3] if i is None else sets[i]
            rot[0] += 1
            torch.matmul(torch.matmul(x, wu.t()), wd.t())

        t = {"inv_warm": median_us(torch, lambda: inv_pair(0)), "inv_rotated": median_us(torch, inv_pair),
             "leaves1_warm": median_us(torch, lambda: inv_pair(0, cn)),
             "hipblaslt_warm": median_us(torch, lambda: fast_pair(0)), "hipblaslt_rotated": median_us(torch, fast_pair)}
        byt = 2.0 * (M * Hd + Ff * Hd + M * Ff) + 2.0 * (M * Ff + Hd * Ff + M * Hd)
        fl = 2.0 * M * (Hd * Ff + Ff * Hd)
        r = {k: round(v, 2) for k, v in t.items()}
        r["inv_rotated_pct_hbm"] = round(100 * byt / (t["inv_rotated"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 1)
        r["inv_warm_tflops"] = round(fl / (t["inv_warm"] * 1e-6) / 1e12, 1)
        r["overhead_vs_hipblaslt_rotated"] = round(t["inv_rotated"] / t["hipblaslt_rotated"] - 1.0, 3)
        dn[f"M={M}"] = r
    out["gemm_dense_pair_us"] = dn
    del sets
    # RMSNorm latency at the dense batch sizes
    out["rmsnorm_us"] = {f"M={M}": round(median_us(torch, lambda: inv.rmsnorm(X[:M], gamma, cn)), 2)
                         for M in (1, 7, 64, 512, 4096)}
    # decode attention at batch prefixes (the same 16 splits at every B)
    if att is not None:
        ar = {}
        cu = att["cu_seqlens"]
        for B in (1, 8, 64):
            L = int(cu[B])
            q = att["q"][:B]
            wsb = inv.attn_workspace(q, ca)
            us = median_us(torch, lambda: inv.decode_attn(q, att["k"][:L], att["v"][:L], cu[:B + 1], att["q_seq"][:B],
                                                          att["q_pos"][:B], ca, ws=wsb))
            ar[f"B={B}"] = {"us": round(us, 2), "kv_tokens": L,
                            "pct_hbm": round(100 * 4096.0 * L / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 1)}
        out["decode_attn"] = ar
    # the MoE layer over contiguous token splits (weights re-read per split)
    if moe is not None:
        T = moe["x"].shape[0]
        mr = {}
        for S in (4, 16):
            n = T // S

            def split_layer():
                for i in range(S):
                    inv.moe_layer(moe["x"][i * n:(i + 1) * n], moe["logits"][i * n:(i + 1) * n],
                                  moe["W1"], moe["W2"], c8, c8)
            mr[f"splits={S}"] = round(median_us(torch, split_layer, iters=10, warm=2) / 1e3, 4)
        out["moe_ms"] = mr
    # LM head + selected-token logprob at small batch: HBM-bound on the 1.24 GB vocabulary matrix
    if lm is not None:
        W, V = lm["W"], lm["W"].shape[0]
        c8f, c64 = inv.contract(leaves=8, out="fp32"), inv.contract(leaves=64)
        lr = {}
        for M in (1, 64):
            h, tg = lm["h"][:M], lm["targets"][:M]
            logits = torch.empty((M, V), dtype=torch.float32, device=dev)
            ws = inv.block16_workspace(M, V, dev)
            gws = torch.empty(max(inv.workspace_bytes(c8f, inv.OP_GEMM, M, V, W.shape[1]), 1), dtype=torch.uint8,
                              device=dev)

            def unfused():
                inv.gemm(h, W, c8f, out=logits, ws=gws)
                inv.logprob(logits, tg, c64)

            def fast():
                torch.log_softmax(torch.matmul(h, W.t()).float(), -1).gather(1, tg.long()[:, None])
            t = {"unfused": median_us(torch, unfused, iters=10, warm=3),
                 "fused": median_us(torch, lambda: inv.lmhead_logprob(h, W, tg, c8f, ws=ws), iters=10, warm=3),
                 "fast_path": median_us(torch, fast, iters=10, warm=3)}
            wbytes = 2.0 * V * W.shape[1]
            r = {k: round(v, 1) for k, v in t.items()}
            r["fused_pct_hbm"] = round(100 * wbytes / (t["fused"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 1)
            r["fused_tokens_per_s"] = round(M / (t["fused"] * 1e-6), 1)
            lr[f"M={M}"] = r
            del logits, ws, gws
        out["lmhead_logprob_us"] = lr
    # copy ceiling (context for the HBM-bound rows)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    cus = median_us(torch, lambda: dst.copy_(src), iters=10, warm=2)
    out["copy_1GiB_gbs"] = round(2.0 * (1 << 30) / (cus * 1e-6) / 1e9, 1)
    del src, dst
    return out


def cpu_baseline(dense_X, W_up, W_down, target_s=12.0):
    """The oracle's 8-leaf GEMM schedule on a bounded row sample of both dense
    projections (TFLOP/s of useful GEMM work, the unit of ``value``). A 32-row
    probe sizes the sample to about ``target_s`` seconds of host work."""
    from threadpoolctl import threadpool_info

    from oracle import gemm as ogemm
    Wu = W_up.float().cpu().numpy()
    Wd = W_down.float().cpu().numpy()

    def run(rows):
        X = dense_X[:rows].float().cpu().numpy()
        t0 = time.perf_counter()
        y = ogemm.gemm_tree(X, Wu, 8, "bf16")
        ogemm.gemm_tree(y, Wd, 8, "bf16")
        return time.perf_counter() - t0

    # whole passes over a row sample until about target_s of host work is done
    probe = run(32)
    rows = int(max(32, min(dense_X.shape[0], 32 * 4.0 / max(probe, 1e-3))))
    rows -= rows % 32
    dt, reps = 0.0, 0
    while dt < target_s and reps < 50:
        dt += run(rows)
        reps += 1
    rows_done = rows * reps
    flops = 2.0 * rows_done * (W_up.shape[0] * W_up.shape[1] + W_down.shape[0] * W_down.shape[1])
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(flops / dt / 1e12, 4), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} pass(es) of {rows} of {dense_X.shape[0]} token rows through both dense "
                      f"projections (4096->12288->4096), 8-leaf fp32 tree schedule with float64 leaf "
                      f"sums, {dt:.1f} s"}


def _cmp(torch, a, b):
    """(elements compared, mismatched elements, max |a - b|) of two tensors of
    one dtype, bit patterns compared (NaN equals NaN only with the same bits)."""
    if a.dtype == torch.bfloat16:
        neq = a.view(torch.int16) != b.view(torch.int16)
    elif a.dtype == torch.float32:
        neq = a.view(torch.int32) != b.view(torch.int32)
    else:
        neq = a != b
    d = (a.float() - b.float()).abs().nan_to_num(0.0)
    return int(a.numel()), int(neq.sum()), float(d.max()) if a.numel() else 0.0


class Tally:
    """Mismatch counts per invariance check, summed over its comparisons."""

    def __init__(self, torch):
        self.torch = torch
        self.rows = {}

    def add(self, name, a, b, what=""):
        n, bad, dmax = _cmp(self.torch, a, b)
        r = self.rows.setdefault(name, {"compared": 0, "mismatched": 0, "max_abs_diff": 0.0, "cases": []})
        r["compared"] += n
        r["mismatched"] += bad
        r["max_abs_diff"] = max(r["max_abs_diff"], dmax)
        if what and what not in r["cases"]:
            r["cases"].append(what)

    def report(self):
        tot = sum(r["compared"] for r in self.rows.values())
        bad = sum(r["mismatched"] for r in self.rows.values())
        return {"elements_compared": tot, "elements_mismatched": bad, "checks": self.rows}


def invariance(torch, inv, synth, step, last, ctx, stages, repeats=20):
    """Bitwise invariance of the step's outputs, GPU against GPU, counted:
    batch size (prefixes and single rows vs the 4096-token batch), emulated
    rank partitions of the GEMM leaves, split-KV rank partitions, prefill vs
    decode, MoE token splits, and ``repeats`` more whole steps against the
    timed run's last step."""
    tl = Tally(torch)
    dev = ctx["dev"]
    if "lmhead" in stages:
        lm, gamma, lp_full = ctx["lm"], ctx["gamma"], last["logprob"]
        c8f, c64, cn = inv.contract(leaves=8, out="fp32"), inv.contract(leaves=64), inv.contract(leaves=1)
        for M in (1, 7, 64, 512):
            hn = inv.rmsnorm(lm["h"][:M].contiguous(), gamma, cn)
            lg = inv.gemm(hn, lm["W"], c8f)
            tl.add("logprob_batch_vs_4096", inv.logprob(lg, lm["targets"][:M].contiguous(), c64), lp_full[:M],
                   f"M={M} prefix")
            del lg
        for i in (1000, 4095):
            hn = inv.rmsnorm(lm["h"][i:i + 1].contiguous(), gamma, cn)
            lg = inv.gemm(hn, lm["W"], c8f)
            tl.add("logprob_batch_vs_4096", inv.logprob(lg, lm["targets"][i:i + 1].contiguous(), c64),
                   lp_full[i:i + 1], f"row {i} alone")
    if "dense" in stages:
        X, W_up, W_down, gamma, b_full = ctx["X"], ctx["W_up"], ctx["W_down"], ctx["gamma"], last["dense"]
        cn = inv.contract(leaves=1)
        yx = inv.rmsnorm(X, gamma, cn)
        a_full = inv.gemm(yx, W_up, inv.contract(leaves=8))
        for R in (2, 4, 8):
            cr = inv.contract(leaves=8, ranks=R)
            tl.add("dense_gemm_rank_partitions", inv.gemm(yx, W_up, cr), a_full, f"R={R} (4096x12288x4096)")
            tl.add("dense_gemm_rank_partitions", inv.gemm(a_full, W_down, cr), b_full, f"R={R} (4096x4096x12288)")
        for M in (1, 7, 64, 512):
            am = inv.gemm(yx[:M].contiguous(), W_up, inv.contract(leaves=8))
            tl.add("dense_batch_vs_4096", inv.gemm(am, W_down, inv.contract(leaves=8)), b_full[:M], f"M={M} prefix")
        del yx, a_full
    if "attn" in stages:
        att, ca, o_full = ctx["att"], ctx["ca"], last["attn"]
        for R in (2, 4, 8):
            ws = inv.attn_workspace(att["q"], ca)
            for r in range(R):
                inv.attn_splits(att["q"], att["k"], att["v"], att["cu_seqlens"], att["q_seq"], att["q_pos"],
                                r * 16 // R, (r + 1) * 16 // R, ca, ws)
            tl.add("attn_split_kv_rank_partitions", inv.attn_combine(ws, att["q"].shape[0], 32, 128, ca), o_full,
                   f"R={R}")
        cu = att["cu_seqlens"]
        for B in (1, 8, 64):
            L = int(cu[B])
            o = inv.decode_attn(att["q"][:B].contiguous(), att["k"][:L], att["v"][:L], cu[:B + 1], att["q_seq"][:B],
                                att["q_pos"][:B], ca)
            tl.add("attn_batch_vs_256", o, o_full[:B], f"B={B} prefix")
        # prefill vs decode: each of 8 sequences as a prefill block of its last 48 positions (the last row's
        # query is the decode query); the decode rows must equal the prefill block's last rows
        qp_all, seq_all, q_all = [], [], []
        for sidx in range(8):
            Ls = int(cu[sidx + 1] - cu[sidx])
            pos = torch.arange(max(0, Ls - 48), Ls, dtype=torch.int32, device=dev)
            qb = synth.randn((pos.numel(), 32, 128), 777 + sidx, device=dev)
            qb[-1] = att["q"][sidx]
            q_all.append(qb)
            qp_all.append(pos)
            seq_all.append(torch.full_like(pos, sidx))
        qpre = torch.cat(q_all).contiguous()
        opre = inv.decode_attn(qpre, att["k"], att["v"], cu, torch.cat(seq_all), torch.cat(qp_all), ca)
        lastrow = torch.cumsum(torch.tensor([q.shape[0] for q in q_all], device=dev), 0) - 1
        tl.add("attn_prefill_vs_decode", opre[lastrow], o_full[:8], "8 sequences, 48-row prefill blocks")
    if "moe" in stages:
        moe, m_full = ctx["moe"], last["moe"]
        c8 = inv.contract(leaves=8)
        T = moe["x"].shape[0]
        for S in (4, 16):
            n = T // S
            parts = [inv.moe_layer(moe["x"][i * n:(i + 1) * n].contiguous(),
                                   moe["logits"][i * n:(i + 1) * n].contiguous(), moe["W1"], moe["W2"], c8, c8)
                     for i in range(S)]
            tl.add("moe_token_splits", torch.cat(parts), m_full, f"{S} splits vs 1")
            del parts
    if "gdn" in stages:
        cg = inv.contract(kv_chunk=64, out="bf16")
        gd = synth.gdn([2048] * 2, H=16, seed=3, device=dev)
        full = inv.gdn_prefill(gd["q"], gd["k"], gd["v"], gd["g"], gd["beta"], gd["cu_seqlens"], cg)
        for P in (1000, 1024):   # prefill P tokens of each sequence, then decode the rest token by token
            cu2 = torch.tensor([0, P, 2 * P], dtype=torch.int32, device=dev)
            idx = torch.cat([torch.arange(0, P, device=dev), torch.arange(2048, 2048 + P, device=dev)])
            cache = inv.gdn_cache(cg, 2, 16, dev)
            inv.gdn_prefill(gd["q"][idx].contiguous(), gd["k"][idx].contiguous(), gd["v"][idx].contiguous(),
                            gd["g"][idx].contiguous(), gd["beta"][idx].contiguous(), cu2, cg, cache=cache)
            outs = []
            for t in range(P, P + 64):
                ti = torch.tensor([t, 2048 + t], device=dev)
                pos = torch.full((2,), t, dtype=torch.int32, device=dev)
                outs.append(inv.gdn_decode(gd["q"][ti].contiguous(), gd["k"][ti].contiguous(),
                                           gd["v"][ti].contiguous(), gd["g"][ti].contiguous(),
                                           gd["beta"][ti].contiguous(), pos, cache, cg))
            dec = torch.stack(outs, 1)  # [2, 64, H, 128]
            ref = torch.stack([full[P:P + 64], full[2048 + P:2048 + P + 64]])
            tl.add("gdn_prefill_then_decode_vs_prefill", dec, ref, f"prefill {P} + 64 decode tokens")
    base = {k: v.clone() for k, v in last.items()}
    for _ in range(repeats):
        o = step()
        for k in base:
            tl.add("repeated_steps", o[k], base[k], f"{repeats} more steps: {', '.join(sorted(base))}")
    torch.cuda.synchronize()
    rep = tl.report()
    rep["repeats"] = repeats
    return rep


def cpu_oracle_configs(ctx, stages, budget_s=3.0):
    """The oracle as it stands, timed end to end per configuration on bounded
    samples of the same inputs (each about ``budget_s`` seconds or one pass)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention as oatt
    from oracle import gemm as ogemm
    from oracle import logprob as olp
    from oracle import moe as omoe
    from oracle import rmsnorm as orms
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    out = {"cores": threads, "kind": "oracle"}

    def timed(fn):
        t0 = time.perf_counter()
        n = 0
        while True:
            fn()
            n += 1
            dt = time.perf_counter() - t0
            if dt >= budget_s or n >= 20:
                return dt / n

    if "dense" in stages or "norm" in stages:
        x = ctx["X"][:512].float().cpu().numpy()
        g = ctx["gamma"].float().cpu().numpy()
        t = timed(lambda: orms.rmsnorm(x, g, 1e-6))
        out["rmsnorm"] = {"tokens_per_s": round(512 / t, 1), "gbs": round(512 * 4 * 4096 / t / 1e9, 4),
                          "sample": "512 rows x 4096, fp64 definition + bf16 cast"}
    if "lmhead" in stages:
        lm = ctx["lm"]
        W = lm["W"]
        V, K = W.shape
        h = lm["h"][:4].float().cpu().numpy()
        blk = 16384
        Wb = W[:blk].float().cpu().numpy()
        t = timed(lambda: ogemm.gemm_tree(h, Wb, 8, "fp32"))
        per_tok = t * V / blk / 4
        out["lm_head_gemm"] = {"tokens_per_s": round(1.0 / per_tok, 4),
                               "tflops": round(2.0 * 4 * blk * K / t / 1e12, 5),
                               "sample": f"4 rows x {blk} of {V} vocabulary rows, 8-leaf fp32 tree schedule "
                                         f"(float64 leaves); per-token rate scaled to the full vocabulary"}
        rng = np.random.default_rng(0)
        lg = rng.normal(size=(64, V)) * 1.3
        tg = rng.integers(0, V, size=64)
        t = timed(lambda: (olp.logprob(lg, tg), olp.merge_tree(*olp.chunk_stats(lg, 64))))
        out["logprob"] = {"tokens_per_s": round(64 / t, 2), "gbs": round(64 * 4.0 * V / t / 1e9, 4),
                          "sample": f"64 rows x {V} logits: plain fp64 definition + the 64-chunk tree"}
    if "attn" in stages:
        att = ctx["att"]
        cu = att["cu_seqlens"].cpu()
        B = 2
        L = int(cu[B])
        q = att["q"][:B].float().cpu().numpy()
        k = att["k"][:L].float().cpu().numpy()
        v = att["v"][:L].float().cpu().numpy()
        t = timed(lambda: oatt.attention(q, k, v, cu[:B + 1].numpy(), att["q_seq"][:B].cpu().numpy(),
                                         att["q_pos"][:B].cpu().numpy(), 8))
        out["decode_attn"] = {"kv_tokens_per_s": round(L / t, 1), "gbs": round(4096.0 * L / t / 1e9, 4),
                              "sample": f"decode rows of the first {B} sequences ({L} keys), fp64 softmax"}
    if "moe" in stages:
        moe = ctx["moe"]
        Tm = 16

        class _E:
            def __init__(self, W):
                self.W, self.shape = W, tuple(W.shape)

            def __getitem__(self, e):
                return self.W[int(e)].float().cpu().numpy().astype(np.float64)
        x = moe["x"][:Tm].float().cpu().numpy().astype(np.float64)
        lg = moe["logits"][:Tm].double().cpu().numpy()
        t = timed(lambda: omoe.moe_layer(x, lg, _E(moe["W1"]), _E(moe["W2"]), 8))
        out["moe_layer"] = {"tokens_per_s": round(Tm / t, 2),
                            "tflops": round(2.0 * Tm * 8 * (1536 * 2048 + 2048 * 768) / t / 1e12, 5),
                            "sample": f"{Tm} tokens through route, expert FFNs and combine (fp64)"}
    return out


def host_device_query():
    """rocminfo / rocm-smi facts (GPU CU count, max clock, current clocks), read
    by child processes before this process touches the GPU. Skipped under a
    profiler's preloaded tool, which would initialise the GPU in the children."""
    import subprocess
    rec = {}
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        rec["rocm_smi_clocks"] = rec["rocminfo"] = "skipped under a profiler"
        return rec
    for cmd, key in ((["rocm-smi", "--showclocks"], "rocm_smi_clocks"), (["rocminfo"], "rocminfo")):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
            lines = r.stdout.splitlines()
            if key == "rocminfo":
                # the GPU agent's section (rocminfo lists the host CPUs first)
                sec, secs = [], []
                for l in lines:
                    if l.startswith("Agent "):
                        secs.append(sec)
                        sec = []
                    sec.append(l)
                secs.append(sec)
                for sec in secs:
                    if any("gfx950" in l for l in sec):
                        for l in sec:
                            if "Max Clock Freq" in l:
                                rec["max_clock_mhz"] = l.split(":", 1)[1].strip()
                            if "Compute Unit" in l:
                                rec["rocminfo_compute_units"] = l.split(":", 1)[1].strip()
                        break
            else:
                rec[key] = [l.strip() for l in lines if "sclk" in l or "mclk" in l or "fclk" in l][:6]
        except Exception as e:  # the record is context; its absence is reported, not fatal
            rec[key] = f"unavailable: {type(e).__name__}"
    return rec


def device_record(torch, inv, host_rec):
    """CU count, clocks and the MFMA ceiling of the device the run used."""
    p = torch.cuda.get_device_properties(0)
    rec = {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
           "hbm_gib": round(p.total_memory / 2 ** 30, 1)}
    rec.update(host_rec)
    # the MFMA ceiling: register-only chains of the path's bf16 instruction, 4 workgroups per CU
    groups, iters = 4 * p.multi_processor_count, 6000
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        clk, fl = inv.bench_mfma_loop(iters, groups)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        c = clk.cpu().double()
        mhz = float((c[:, 0] / c[:, 1]).median() * 100.0)
        if best is None or ms < best[0]:
            best = (ms, fl, mhz)
    ms, fl, mhz = best
    rec["mfma_ceiling"] = {"tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                           "frac_of_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "shader_clock_mhz_during_loop": round(mhz, 1),
                           "kernel": "8 waves per workgroup, 8 independent v_mfma_f32_16x16x32_bf16 chains "
                                     "per wave, register operands only"}
    return rec


def recorded_traffic():
    """HBM bytes per dense GEMM launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel's reading), or
    None when gemm.hip has changed since those counters were taken."""
    import hashlib
    summ = os.path.join(ROOT, "profiles", "gemm_dense_traffic.md")
    src = os.path.join(ROOT, "split_invariant_deterministic_amd", "csrc", "gemm.hip")
    if not os.path.exists(summ):
        return None
    vals = {}
    for line in open(summ):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if vals.get("gemm.hip sha256") != sha or "traffic bytes per launch" not in vals:
        return None
    return float(vals["traffic bytes per launch"])


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; multi-GPU sharding is a design "
                                   "note (no collectives are built), run with --gpus 1"}))
        sys.exit(2)
    host_rec = host_device_query()  # child processes, before this process initialises the GPU
    import torch
    import torch.nn.functional as F

    from split_invariant_deterministic_amd import inv, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stages = set(args.stages.split(","))
    T = Timer(torch)

    # ------------------------------------------------------------ inputs (HBM-resident)
    M, Hd, Ff = 4096, 4096, 12288
    dense = synth.dense(Hd, Ff, M=M, seed=0, device=dev)
    X, W_up = dense["X"], dense["W"]
    W_down = synth.dense(Ff, Hd, M=1, seed=1, device=dev)["W"]
    gamma = synth.rmsnorm(1, Hd, seed=0, device=dev)["gamma"]
    c8 = inv.contract(leaves=8)
    c8f = inv.contract(leaves=8, out="fp32")
    cn = inv.contract(leaves=1)
    c64 = inv.contract(leaves=64)
    if "norm" in stages:
        xn = synth.rmsnorm(65536, Hd, seed=1, device=dev)["x"]
        yn = torch.empty_like(xn)
    if "copy" in stages:
        csrc = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)
    if "attn" in stages:
        lengths = synth.attn_lengths(256, 32768, seed=0)
        att = synth.attn(lengths, seed=0, device=dev)
        for k in ("cu_seqlens", "q_seq", "q_pos"):
            att[k] = att[k].to(dev)
        ca = inv.contract()
        att_ws = inv.attn_workspace(att["q"], ca)
        sumL = int(lengths.sum())
    if "moe" in stages:
        moe = synth.moe(T=8192, seed=0, device=dev)
    if "lmhead" in stages:
        lm = synth.lmhead(M=M, seed=0, device=dev)
        logits = torch.empty((M, lm["W"].shape[0]), dtype=torch.float32, device=dev)
    log("inputs resident")
    y = torch.empty_like(X)
    a = torch.empty((M, Ff), dtype=torch.bfloat16, device=dev)
    b = torch.empty((M, Hd), dtype=torch.bfloat16, device=dev)

    def step():
        outs = {}
        if "dense" in stages:
            T.start("rmsnorm")
            inv.rmsnorm(X, gamma, cn, out=y)
            T.stop("rmsnorm")
            T.start("gemm_dense")
            inv.gemm(y, W_up, c8, out=a)
            inv.gemm(a, W_down, c8, out=b)
            T.stop("gemm_dense")
            outs["dense"] = b
        if "norm" in stages:
            T.start("rmsnorm_bw")
            inv.rmsnorm(xn, gamma, cn, out=yn)
            T.stop("rmsnorm_bw")
        if "copy" in stages:
            T.start("copy")
            cdst.copy_(csrc)
            T.stop("copy")
        if "attn" in stages:
            T.start("attn")
            outs["attn"] = inv.decode_attn(att["q"], att["k"], att["v"], att["cu_seqlens"], att["q_seq"],
                                           att["q_pos"], ca, ws=att_ws)
            T.stop("attn")
        if "moe" in stages:
            T.start("moe")
            outs["moe"] = inv.moe_layer(moe["x"], moe["logits"], moe["W1"], moe["W2"], c8, c8)
            T.stop("moe")
        if "lmhead" in stages:
            T.start("lm_rmsnorm")
            hn = inv.rmsnorm(lm["h"], gamma, cn)
            T.stop("lm_rmsnorm")
            T.start("gemm_lmhead")
            inv.gemm(hn, lm["W"], c8f, out=logits)
            T.stop("gemm_lmhead")
            T.start("logprob")
            outs["logprob"] = inv.logprob(logits, lm["targets"], c64)
            T.stop("logprob")
        return outs

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")
    T.reset()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        T.start("step")
        last = step()
        T.stop("step")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {k: T.mean_ms(k) for k in T.ev}
    ms_step = wall * 1e3 / args.steps
    log(f"timed steps done: {ms_step:.2f} ms/step")

    # ------------------------------------------------------------ fused LM head (outside the step)
    # The same LM head with the logprob reduced in the GEMM epilogue (16-column
    # vocabulary blocks, logits never stored): timed beside the step's unfused
    # GEMM + logprob, not added to it.
    if "lmhead" in stages:
        V = lm["W"].shape[0]
        lm_ws = inv.block16_workspace(M, V, dev)
        hn = inv.rmsnorm(lm["h"], gamma, cn)
        Tx = Timer(torch)
        for i in range(max(3, min(args.steps, 10)) + 2):
            if i == 2:
                torch.cuda.synchronize()
                Tx.reset()
            Tx.start("lmhead_fused")
            inv.lmhead_logprob(hn, lm["W"], lm["targets"], c8f, ws=lm_ws)
            Tx.stop("lmhead_fused")
        torch.cuda.synchronize()
        ms["lmhead_fused"] = Tx.mean_ms("lmhead_fused")
        del lm_ws
        log("fused LM head timed")

    # ------------------------------------------------------------ CPR Gated DeltaNet (outside the step)
    # Prefill of 5 sequences x 2048 tokens, 16 heads of width 128, chunk 64; one
    # decode token for 256 sequences, once at a plain position and once at a
    # position that closes a chunk (the boundary update and resynchronisation).
    if "gdn" in stages:
        cg = inv.contract(kv_chunk=64, out="bf16")
        gd = synth.gdn([2048] * 5, H=16, seed=0, device=dev)
        Tg = gd["q"].shape[0]
        g_ws = torch.empty(inv.workspace_bytes(cg, inv.OP_GDN_PREFILL, Tg, 16, 5), dtype=torch.uint8, device=dev)
        g_out = torch.empty((Tg, 16, 128), dtype=torch.bfloat16, device=dev)
        dq = synth.gdn([1] * 256, H=16, seed=1, device=dev)
        g_cache = inv.gdn_cache(cg, 256, 16, dev)
        d_out = torch.empty((256, 16, 128), dtype=torch.bfloat16, device=dev)
        pos_plain = torch.full((256,), 2048, dtype=torch.int32, device=dev)
        pos_close = torch.full((256,), 2111, dtype=torch.int32, device=dev)
        Tx = Timer(torch)
        for i in range(max(3, min(args.steps, 10)) + 2):
            if i == 2:
                torch.cuda.synchronize()
                Tx.reset()
            Tx.start("gdn_prefill")
            inv.gdn_prefill(gd["q"], gd["k"], gd["v"], gd["g"], gd["beta"], gd["cu_seqlens"], cg, out=g_out, ws=g_ws)
            Tx.stop("gdn_prefill")
            Tx.start("gdn_decode")
            inv.gdn_decode(dq["q"], dq["k"], dq["v"], dq["g"], dq["beta"], pos_plain, g_cache, cg, out=d_out)
            Tx.stop("gdn_decode")
            Tx.start("gdn_decode_boundary")
            inv.gdn_decode(dq["q"], dq["k"], dq["v"], dq["g"], dq["beta"], pos_close, g_cache, cg, out=d_out)
            Tx.stop("gdn_decode_boundary")
        torch.cuda.synchronize()
        for k in ("gdn_prefill", "gdn_decode", "gdn_decode_boundary"):
            ms[k] = Tx.mean_ms(k)
        del g_ws, gd, g_cache
        log("CPR Gated DeltaNet timed")

    # ------------------------------------------------------------ shape sweep (outside the step)
    sw = None
    if "sweep" in stages:
        sw = sweep(torch, inv, synth, X, W_up, W_down, gamma, att if "attn" in stages else None,
                   moe if "moe" in stages else None, lm if "lmhead" in stages else None, c8, cn,
                   ca if "attn" in stages else None, dev)
        log("shape sweep done")

    # ------------------------------------------------------------ invariance (outside the timed steps)
    ctx = {"dev": dev, "X": X, "W_up": W_up, "W_down": W_down, "gamma": gamma}
    if "lmhead" in stages:
        ctx["lm"] = lm
    if "attn" in stages:
        ctx.update(att=att, ca=ca)
    if "moe" in stages:
        ctx["moe"] = moe
    inv_rep = None
    if args.invariance_repeats >= 0:
        inv_rep = invariance(torch, inv, synth, step, last, ctx, stages, repeats=args.invariance_repeats)
        log(f"invariance: {inv_rep['elements_mismatched']} of {inv_rep['elements_compared']} elements differ")
    dev_rec = device_record(torch, inv, host_rec)
    log("device record and MFMA ceiling done")

    # ------------------------------------------------------------ fast paths
    Tf = Timer(torch)
    fast = {}
    reps = max(3, min(args.steps, 10))
    for i in range(reps + 2):
        if i == 2:
            torch.cuda.synchronize()
            Tf.reset()
        if "dense" in stages:
            Tf.start("rmsnorm")
            yf = F.rms_norm(X, (Hd,), gamma, 1e-6)
            Tf.stop("rmsnorm")
            Tf.start("gemm_dense")
            af = torch.matmul(yf, W_up.t())
            torch.matmul(af, W_down.t())
            Tf.stop("gemm_dense")
        if "norm" in stages:
            Tf.start("rmsnorm_bw")
            F.rms_norm(xn, (Hd,), gamma, 1e-6)
            Tf.stop("rmsnorm_bw")
        if "lmhead" in stages:
            Tf.start("logprob")
            torch.log_softmax(logits, -1).gather(1, lm["targets"].long()[:, None])
            Tf.stop("logprob")
            Tf.start("gemm_lmhead")
            torch.matmul(lm["h"], lm["W"].t())
            Tf.stop("gemm_lmhead")
        if "attn" in stages:
            # same kernel, split count chosen for occupancy (not invariant across batch sizes)
            cfast = inv.contract(split_kv=4)
            Tf.start("attn")
            inv.decode_attn(att["q"], att["k"], att["v"], att["cu_seqlens"], att["q_seq"], att["q_pos"], cfast,
                            ws=att_ws)
            Tf.stop("attn")
    torch.cuda.synchronize()
    fast = {k: Tf.mean_ms(k) for k in Tf.ev}
    overhead = {k: (ms[k] / fast[k] - 1.0) for k in fast if k in ms and fast[k] > 0}

    # ------------------------------------------------------------ metric + roofline
    result = {
        "metric": "invariant GEMM TFLOP/s (% MFMA peak) + logprob tokens/s; overhead vs fast path",
        "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights; no dataset, no weights)",
        "config": {"workload": "dense 8B-class projections 4096->12288->4096 at M=4096 tokens, 8 K-leaves "
                               "(+ split-KV decode attention B=256, MoE 8192 tokens, LM head 4096x151936 "
                               "with 64-chunk logprob in the same step)",
                   "global_batch": M, "seq_len": 1, "parallelism": "none (1 GPU)"},
    }
    if "dense" in stages:
        flops = 2.0 * M * (Hd * Ff + Ff * Hd)
        tflops = flops / (ms["gemm_dense"] * 1e-3) / 1e12
        result["value"] = round(tflops, 2)
        result["pct_mfma_peak"] = round(100 * tflops / PEAK_BF16_TFLOPS, 2)
        result["roofline"] = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                              "traffic": recorded_traffic(),
                              "kernel": "inv_gemm (gemm_ring_kernel<8, 64, bf16>), 4096x12288x4096 + 4096x4096x12288, "
                                        "2*M*N*K flops per launch over the mean launch time"}
        result["rmsnorm_gbs"] = round(2 * 2 * M * Hd / (ms["rmsnorm"] * 1e-3) / 1e9, 1)
    if "lmhead" in stages:
        V = lm["W"].shape[0]
        result["logprob_tokens_per_s"] = round(M / (ms["logprob"] * 1e-3), 1)
        result["logprob_gbs"] = round(4.0 * V * M / (ms["logprob"] * 1e-3) / 1e9, 1)
        result["logprob_pct_hbm"] = round(100 * result["logprob_gbs"] / PEAK_HBM_GBS, 2)
        lm_ms = ms["lm_rmsnorm"] + ms["gemm_lmhead"] + ms["logprob"]
        result["lmhead_logprob_tokens_per_s"] = round(M / (lm_ms * 1e-3), 1)
        result["gemm_lmhead_tflops"] = round(2.0 * M * V * Hd / (ms["gemm_lmhead"] * 1e-3) / 1e12, 2)
        fused_ms = ms["lm_rmsnorm"] + ms["lmhead_fused"]
        result["lmhead_fused_logprob_tokens_per_s"] = round(M / (fused_ms * 1e-3), 1)
        result["lmhead_fused_speedup"] = round(lm_ms / fused_ms, 3)
    if "attn" in stages:
        result["attn_gbs"] = round(4096.0 * sumL / (ms["attn"] * 1e-3) / 1e9, 1)
    if "gdn" in stages:
        result["gdn_prefill_tokens_per_s"] = round(10240 / (ms["gdn_prefill"] * 1e-3), 1)
        result["gdn_prefill_ms"] = round(ms["gdn_prefill"], 4)
        result["gdn_decode_ms"] = round(ms["gdn_decode"], 4)
        result["gdn_decode_boundary_ms"] = round(ms["gdn_decode_boundary"], 4)
    if "moe" in stages:
        result["moe_tflops"] = round(2.0 * 8192 * 8 * (1536 * 2048 + 2048 * 768) / (ms["moe"] * 1e-3) / 1e12, 2)
    if "norm" in stages:
        result["rmsnorm_bw_gbs"] = round(2 * 2 * 65536 * Hd / (ms["rmsnorm_bw"] * 1e-3) / 1e9, 1)
    if "copy" in stages:
        result["copy_gbs"] = round(2.0 * (1 << 30) / (ms["copy"] * 1e-3) / 1e9, 1)
    # every kernel against its own roofline: algorithmic work per unit x units per launch
    rl = {}

    def add(name, bound, work, t_ms, peak, unit):
        a = work / (t_ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        rl[name] = {"bound": bound, "achieved": round(a, 1), "peak": peak, "unit": unit, "frac": round(a / peak, 4)}

    if "dense" in stages:
        add("inv_gemm dense (2 launches)", "mfma", 2.0 * M * (Hd * Ff + Ff * Hd), ms["gemm_dense"],
            PEAK_BF16_TFLOPS, "TFLOP/s")
    if "norm" in stages:
        add("inv_rmsnorm 65536x4096", "hbm", 4.0 * 65536 * Hd, ms["rmsnorm_bw"], PEAK_HBM_GBS, "GB/s")
    if "lmhead" in stages:
        add("inv_gemm lm head", "mfma", 2.0 * M * V * Hd, ms["gemm_lmhead"], PEAK_BF16_TFLOPS, "TFLOP/s")
        add("inv_logprob 4096x151936", "hbm", 4.0 * V * M, ms["logprob"], PEAK_HBM_GBS, "GB/s")
        add("inv_lmhead_logprob (fused) 4096x151936x4096", "mfma", 2.0 * M * V * Hd, ms["lmhead_fused"],
            PEAK_BF16_TFLOPS, "TFLOP/s")
    if "attn" in stages:
        add("inv_decode_attn B=256", "hbm", 4096.0 * sumL, ms["attn"], PEAK_HBM_GBS, "GB/s")
    if "gdn" in stages:
        # CPR flops per (token, head): the recurrence step 7*128^2 (S^T k, the
        # rank-1 update with decay, S^T q) plus the chunk update amortised over
        # C = 64 tokens, (4*128^2*C + 2*C*(C-1)*128) / C. fp32 throughout: the
        # recurrence on vector FMAs, the chunk update on fp32 MFMA; both peak at
        # 157.3 TFLOP/s on MI355X.
        fl_tok = 7 * 128 * 128 + (4 * 128 * 128 * 64 + 2 * 64 * 63 * 128) / 64
        add("gdn prefill 5x2048 tokens, 16 heads", "alu", fl_tok * 10240 * 16, ms["gdn_prefill"],
            PEAK_FP32_TFLOPS, "TFLOP/s")
        # decode: the running state read and written, 2 * 128^2 * 4 bytes per (sequence, head)
        add("gdn decode 256 sequences, 16 heads", "hbm", 2 * 128 * 128 * 4 * 256 * 16, ms["gdn_decode"],
            PEAK_HBM_GBS, "GB/s")
    if "moe" in stages:
        add("moe layer 8192 tokens", "mfma", 2.0 * 8192 * 8 * (1536 * 2048 + 2048 * 768), ms["moe"],
            PEAK_BF16_TFLOPS, "TFLOP/s")
    result["rooflines"] = rl
    if sw is not None:
        result["sweep"] = sw
    if inv_rep is not None:
        result["invariance"] = inv_rep
    result["device"] = dev_rec
    result["stage_ms"] = {k: round(v, 4) for k, v in ms.items()}
    result["fast_ms"] = {k: round(v, 4) for k, v in fast.items()}
    result["overhead_vs_fast"] = {k: round(v, 3) for k, v in overhead.items()}
    log("fast paths done")
    if not args.no_cpu_baseline and "dense" in stages:
        log("timing the CPU oracle on a row sample")
        result["cpu_baseline"] = cpu_baseline(X, W_up, W_down)
        log("timing the CPU oracle per configuration")
        result["cpu_oracle_configs"] = cpu_oracle_configs(ctx, stages)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
