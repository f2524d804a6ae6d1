"""Rounding to the storage precisions (test infrastructure; see oracle/__init__).

The pages fix no rounding points; the readings used here: inputs, stored
compressed entries, the normalised query and the normalised window keys and
the final output are rounded to the storage type (bf16 or fp32); everything
else is carried in float64.
"""
import numpy as np


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits.  With x = f * 2**e and 0.5 <= |f| < 1
    (numpy.frexp), the nearest bf16 value is rint(f * 2**8) * 2**(e - 8);
    numpy.rint rounds halves to even.  Values here are far from the bf16
    overflow and subnormal ranges.
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    return np.ldexp(np.rint(f * 256.0), e - 8)


def round_f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to(x, dtype: str):
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return round_f32(x)
    raise ValueError(dtype)
