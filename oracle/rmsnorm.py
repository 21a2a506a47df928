"""RMSNorm over the hidden dimension (oracle side).

[RLK] section 4 lists RMSNorm as the reduction class over the hidden
dimension; [RLK] section 6 (module 02) and [VeXact] section 3.1 use an RMSNorm
with one fixed semantics on both sides, the latter citing Zhang and Sennrich's
root-mean-square layer normalization:

    y[m, h] = x[m, h] / sqrt( mean_h x[m, h]^2 + eps ) * gamma[h]

computed here in float64 from bf16 inputs and rounded once to bf16 (RNE).
eps is taken as the float32 value the contract stores.

Pinned by: closed forms in the tests (zero row, constant row, single nonzero
element) and an exact rational sum of squares on the tiny shape.
"""

import numpy as np

from . import numerics


def rmsnorm(x, gamma, eps=1e-6, rows=None):
    x = np.asarray(x, dtype=np.float64)
    if rows is not None:
        x = x[rows]
    g = np.asarray(gamma, dtype=np.float64)
    eps32 = float(np.float32(eps))
    ms = np.mean(x * x, axis=1)
    r = 1.0 / np.sqrt(ms + eps32)
    return numerics.to_bf16(x * r[:, None] * g[None, :])


def inv_rms(x, eps=1e-6):
    """The float64 scale 1/sqrt(mean x^2 + eps) per row (for localisation)."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=1) + float(np.float32(eps)))
