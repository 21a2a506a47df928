"""Tolerance checks shared by the GPU parity tests.

The bars (the tolerances the invariant path is held to):

* bf16 outputs (GEMM, RMSNorm, attention, MoE): elementwise
  |gpu - ora| <= max(1 bf16 ulp of ora, 2e-3 * rms of the oracle row), and
  normwise ||gpu - ora|| / ||ora|| <= 2e-3. One ulp: 2e-3 relative is finer
  than half a bf16 ulp, so an fp32 value that straddles a rounding midpoint
  legitimately flips one ulp. The row-scale term: an output that cancels to
  near zero carries the fp32 accumulation error of its large terms, which
  no fp32 kernel can hold to one bf16 ulp of a tiny value; 2e-3 of the row's
  scale still fails on any dropped or wrong term (each term of these
  workloads is of order 1e-2 of the row scale or more);
* fp32 GEMM outputs (leaf partials, logits): |gpu - ora| <= 2e-3 *
  max(|ora|, rms of the oracle row);
* fp32 logprobs: |gpu - ora| <= max(1e-5 * |ora|, floor), floor = 4 fp32
  ulps of |LSE| (at least 1e-6): the LSE is formed in fp32 by three rounded
  steps (log2, the ln 2 scale, the add of the maximum), each worth up to about
  one ulp of the LSE's magnitude, and lp = x_t - LSE cannot be finer than
  that. For the near-uniform rows of the LM-head workload (lp ~ -12) the
  relative term is 30x larger than the floor, so only near-zero logprobs of
  peaked rows ever use it.
"""

import numpy as np

from oracle import numerics


def as_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if hasattr(t, "detach") else np.asarray(t)


def check_bf16(gpu, ora, what="", norm_tol=2e-3, scale_tol=2e-3):
    g = as_np(gpu)
    o = np.asarray(ora, dtype=np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    ulp = np.maximum(numerics.bf16_ulp(o), numerics.bf16_ulp(g))  # a flip across a binade edge
    rows = o.reshape(-1, o.shape[-1]) if o.ndim else o.reshape(1, 1)
    rms = np.sqrt(np.mean(rows * rows, axis=-1, keepdims=True)).reshape(o.shape[:-1] + (1,)) if o.ndim else 0.0
    lim = np.maximum(ulp * (1 + 1e-12), scale_tol * rms)
    bad = np.abs(g - o) > lim
    assert not np.any(bad), f"{what}: {int(bad.sum())} elements outside max(1 bf16 ulp, {scale_tol} row rms); " \
                            f"first {np.argwhere(bad)[:4].tolist()} gpu {g[bad][:4]} ora {o[bad][:4]}"
    den = np.linalg.norm(o)
    if den > 0:
        rel = np.linalg.norm(g - o) / den
        assert rel <= norm_tol, f"{what}: normwise error {rel:.3e} > {norm_tol}"
    return int(g.size)


def ulps_off(gpu, ora):
    """Number of elements more than one bf16 ulp from the oracle (reported, not a bar)."""
    g = as_np(gpu)
    o = np.asarray(ora, dtype=np.float64)
    return int(np.sum(np.abs(g - o) > np.maximum(numerics.bf16_ulp(o), numerics.bf16_ulp(g)) * (1 + 1e-12)))


def check_fp32_gemm(gpu, ora, what="", tol=2e-3):
    g = as_np(gpu)
    o = np.asarray(ora, dtype=np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
    lim = tol * np.maximum(np.abs(o), rms)
    bad = np.abs(g - o) > lim
    assert not np.any(bad), f"{what}: {int(bad.sum())} outside {tol}; first {np.argwhere(bad)[:4].tolist()}"
    return int(g.size)


def check_logprob(gpu, ora, what="", lse=None, rel=1e-5, floor=1e-6):
    g = as_np(gpu)
    o = np.asarray(ora, dtype=np.float64)
    assert g.shape == o.shape
    nan_o = np.isnan(o)
    assert np.array_equal(np.isnan(g), nan_o), f"{what}: NaN pattern differs"
    fl = np.full(o.shape, floor)
    if lse is not None:
        a = np.abs(np.asarray(lse, dtype=np.float64)).astype(np.float32)
        fl = np.maximum(fl, 4.0 * np.spacing(a).astype(np.float64))
    lim = np.maximum(rel * np.abs(o), fl)
    bad = (np.abs(g - o) > lim) & ~nan_o
    assert not np.any(bad), f"{what}: {int(bad.sum())} outside; first {np.argwhere(bad)[:4].ravel().tolist()} " \
                            f"gpu {g[bad][:4]} ora {o[bad][:4]} lim {lim[bad][:4]}"
    return int(g.size)


def bitwise_equal(a, b):
    """Bit-pattern equality of two tensors (NaN == NaN if same bits)."""
    import torch
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    if a.dtype in (torch.bfloat16, torch.float16):
        return bool(torch.equal(a.view(torch.int16), b.view(torch.int16)))
    if a.dtype == torch.float32:
        return bool(torch.equal(a.view(torch.int32), b.view(torch.int32)))
    return bool(torch.equal(a, b))


def mismatch_report(a, b):
    """(elements compared, mismatched elements, max abs difference)."""
    import torch
    fa = a.float()
    fb = b.float()
    if a.dtype == torch.bfloat16:
        neq = a.view(torch.int16) != b.view(torch.int16)
    elif a.dtype == torch.float32:
        neq = a.view(torch.int32) != b.view(torch.int32)
    else:
        neq = a != b
    return int(a.numel()), int(neq.sum()), float((fa - fb).abs().nan_to_num(0).max()) if a.numel() else 0.0
