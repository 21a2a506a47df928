"""Split-invariant logprob forward for MI355X (gfx950).

The compute path is the C-ABI library ``libinv.so`` (hand-written HIP
kernels, declared in ``include/inv.h``); ``split_invariant_deterministic_amd.inv``
is its thin ctypes binding over torch device tensors. Importing the package
itself loads nothing, so the seeded input generators in ``synth`` can be used
without the library; importing ``inv`` raises if the library is missing.
"""

__all__ = ["inv", "synth", "build"]
