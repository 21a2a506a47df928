"""Number formats used at the path's precision boundaries (oracle side).

[RLK] section 2 lists the position of the FP32 <-> BF16 conversion as one of
the four trigger points of mismatch; [RLK] section 7 has the ROCm GEMM merge
in FP32 and write BF16 once. The oracle therefore needs an exact
round-to-nearest-even (RNE) cast to bf16 from any float64 value, written here
from the definition of the format (1 sign bit, 8 exponent bits with bias 127,
7 stored significand bits; subnormals below 2**-126; largest finite value
(2 - 2**-7) * 2**127).

Pinned by: tests compare ``to_bf16`` with torch's CPU float32 -> bfloat16
conversion on stratified float32 bit patterns (a library routine), and with
hand-computed ties.
"""

import numpy as np

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_BF16_MIN_ULP_EXP = -133  # ulp of bf16 subnormals: 2**-126 * 2**-7


def to_bf16(v):
    """Round float64 values to the nearest bf16 value, ties to even.

    Returns float64 values that are exactly representable in bf16 (so they
    convert to float32 without change). NaN stays NaN, +-inf stay inf, values
    that round beyond the largest finite bf16 become +-inf, signed zero is
    kept.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.array(v, dtype=np.float64, copy=True)
    finite = np.isfinite(v) & (v != 0.0)
    if np.any(finite):
        x = v[finite]
        _, e = np.frexp(x)  # |x| in [2**(e-1), 2**e)
        ulp_exp = np.maximum(e - 8, _BF16_MIN_ULP_EXP)  # 8 significant bits
        q = np.ldexp(x, -ulp_exp)  # exact power-of-two scaling
        r = np.ldexp(np.rint(q), ulp_exp)  # np.rint rounds half to even
        r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, x), r)
        out[finite] = r
    return out


def bf16_bits(v):
    """uint16 bit patterns of bf16 values (input must already be bf16-exact)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bits_to_float(bits):
    """float32 values of uint16 bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (the ulp of the binade of v)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(np.where(v == 0.0, 2.0 ** -126, v))
    return np.ldexp(1.0, np.maximum(e - 8, _BF16_MIN_ULP_EXP))


def f32(v):
    """Round float64 to float32 (IEEE RNE, numpy's cast)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)
