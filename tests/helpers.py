"""Tolerance checks shared by the GPU parity tests.

The bars (the tolerances the invariant path is held to):

* bf16 outputs (GEMM, RMSNorm, attention, MoE): elementwise the GPU value is
  within one bf16 ulp of the oracle's bf16 value (0.002 relative is finer
  than half a bf16 ulp, so an fp32 difference that straddles a rounding
  midpoint legitimately flips one ulp), and normwise
  ||gpu - ora|| / ||ora|| <= 2e-3;
* fp32 GEMM outputs (leaf partials, logits): |gpu - ora| <= 2e-3 *
  max(|ora|, rms of the oracle row);
* fp32 logprobs: |gpu - ora| <= 1e-5 * |ora|, with an absolute floor of
  1e-6 where |ora| < 0.1.
"""

import numpy as np

from oracle import numerics


def as_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if hasattr(t, "detach") else np.asarray(t)


def check_bf16(gpu, ora, what="", norm_tol=2e-3):
    g = as_np(gpu)
    o = np.asarray(ora, dtype=np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    ulp = numerics.bf16_ulp(o)
    # a flip across a binade edge can land on the next binade's spacing
    bad = np.abs(g - o) > np.maximum(ulp, numerics.bf16_ulp(g)) * (1 + 1e-12)
    assert not np.any(bad), f"{what}: {int(bad.sum())} elements off by more than 1 bf16 ulp; " \
                            f"first {np.argwhere(bad)[:4].tolist()} gpu {g[bad][:4]} ora {o[bad][:4]}"
    den = np.linalg.norm(o)
    if den > 0:
        rel = np.linalg.norm(g - o) / den
        assert rel <= norm_tol, f"{what}: normwise error {rel:.3e} > {norm_tol}"
    return int(g.size)


def check_fp32_gemm(gpu, ora, what="", tol=2e-3):
    g = as_np(gpu)
    o = np.asarray(ora, dtype=np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True))
    lim = tol * np.maximum(np.abs(o), rms)
    bad = np.abs(g - o) > lim
    assert not np.any(bad), f"{what}: {int(bad.sum())} outside {tol}; first {np.argwhere(bad)[:4].tolist()}"
    return int(g.size)


def check_logprob(gpu, ora, what="", rel=1e-5, floor=1e-6):
    g = as_np(gpu)
    o = np.asarray(ora, dtype=np.float64)
    assert g.shape == o.shape
    nan_o = np.isnan(o)
    assert np.array_equal(np.isnan(g), nan_o), f"{what}: NaN pattern differs"
    lim = np.where(np.abs(o) < 0.1, np.maximum(rel * np.abs(o), floor), rel * np.abs(o))
    bad = (np.abs(g - o) > lim) & ~nan_o
    assert not np.any(bad), f"{what}: {int(bad.sum())} outside {rel} rel; worst " \
                            f"{np.max(np.abs(g - o)[~nan_o] / np.maximum(np.abs(o[~nan_o]), 1e-30)):.3e}"
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
