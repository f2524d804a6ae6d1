"""FP8 (E4M3) indexer keys (test infrastructure; see oracle/__init__).

Pages: "DeepSeek-V4", Inference efficiency (the indexer's query-key path runs
in low precision in the released model).  The pages give no format details;
the reading taken here stores the indexer-key cache -- the dominant stream of
a decode step -- at one byte per channel:

* E4M3 is the OCP 8-bit float with 1 sign, 4 exponent (bias 7) and 3
  mantissa bits: normal values (1 + m/8) * 2**(e - 7), subnormals
  m/8 * 2**-6 (spacing 2**-9), largest finite 448, no infinities.
* A key row v is stored as E4M3 values q and one fp32 scale
  s = fp32(max|v| / 448); q = RNE(v / s), limited to [-448, 448] (0 and s = 0
  for an all-zero row).  The row stands for s * q.
* The score of a key under fp8 is the plain score of the row it stands for,
  with the query at its own precision:
      s_j = sum_h omega_h * max(0, p_h . (s_j q_j)).
"""
import numpy as np

from . import indexer
from . import numerics

E4M3_MAX = 448.0


def round_e4m3(x):
    """Nearest E4M3 value of float64 values with |x| <= 448, ties to even.

    Inside a binade [2**b, 2**(b+1)) the E4M3 values are spaced 2**(b-3);
    below 2**-6 (subnormals) the spacing is 2**-9.  Rounding |x| to the
    nearest multiple of its binade's spacing with numpy.rint (halves to the
    even multiple, which is the even mantissa) gives the nearest value; a
    carry to 16 multiples lands on the next binade's first value, which is
    representable.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > E4M3_MAX):
        raise ValueError("round_e4m3: |x| above 448")
    _, e = np.frexp(a)                      # a = f * 2**e, 0.5 <= f < 1: binade 2**(e-1)
    spacing = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    return np.copysign(np.rint(a / spacing) * spacing, x)


def quantize_rows(v):
    """Rows [N, C] -> (q [N, C] E4M3 values as float64, s [N] fp32 scales)."""
    v = np.asarray(v, dtype=np.float64)
    amax = np.max(np.abs(v), axis=-1) if v.shape[-1] else np.zeros(v.shape[:-1])
    s = numerics.round_f32(amax / E4M3_MAX)
    safe = np.where(s > 0, s, 1.0)
    q = round_e4m3(np.clip(v / safe[..., None], -E4M3_MAX, E4M3_MAX))
    q = np.where(s[..., None] > 0, q, 0.0)
    return q, s


def dequantize_rows(q, s):
    return np.asarray(q, dtype=np.float64) * np.asarray(s, dtype=np.float64)[..., None]


def scores_fp8(p, omega, q, s):
    """Indexer scores of fp8 keys (q [N, d_I], s [N]) for the query p
    [H_I, d_I] -> [N] float64."""
    return indexer.scores(p, omega, dequantize_rows(q, s))


# --------------------------------------------------------------------------
# MXFP4 (OCP microscaling FP4) indexer keys
#
# Reading: each block of 32 consecutive channels of a key row shares one E8M0
# scale s = 2**(floor(log2(amax)) - 2) (2 = the largest exponent of E2M1, so
# the block's largest value lands in [4, 8) and is clamped to 6); the elements
# are E2M1 values (1 sign, 2 exponent bits of bias 1, 1 mantissa bit:
# 0, 0.5, 1, 1.5, 2, 3, 4, 6) of v / s, rounded to nearest even and clamped to
# +-6; an all-zero block has scale 2**-127 and zero elements.  The row stands
# for s * q; its score is the plain score of that row.
# --------------------------------------------------------------------------

E2M1_MAX = 6.0
MX_BLOCK = 32


def round_e2m1(x):
    """Nearest E2M1 value of float64 values with |x| <= 6, ties to even: the
    spacing is 0.5 below 2 and 2**(b-1) in the binade [2**b, 2**(b+1)), b >= 1;
    numpy.rint takes halves to the even multiple (the even mantissa)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > E2M1_MAX):
        raise ValueError("round_e2m1: |x| above 6")
    _, e = np.frexp(a)                      # a = f * 2**e, 0.5 <= f < 1: binade 2**(e-1)
    spacing = np.ldexp(1.0, np.maximum(e - 1, 0) - 1)
    return np.copysign(np.rint(a / spacing) * spacing, x)


def quantize_mx_rows(v, block: int = MX_BLOCK):
    """Rows [N, C] (C a multiple of block) -> (q [N, C] E2M1 values, s [N, C/block]
    power-of-two scales)."""
    v = np.asarray(v, dtype=np.float64)
    N, C = v.shape
    vb = v.reshape(N, C // block, block)
    amax = np.max(np.abs(vb), axis=-1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))   # floor(log2(amax)) = e - 1
    ex = np.clip(e - 1 - 2, -127, 127)
    s = np.where(amax > 0, np.ldexp(1.0, ex), 2.0 ** -127)
    q = round_e2m1(np.clip(vb / s[..., None], -E2M1_MAX, E2M1_MAX))
    q = np.where(amax[..., None] > 0, q, 0.0)
    return q.reshape(N, C), s


def dequantize_mx_rows(q, s, block: int = MX_BLOCK):
    q = np.asarray(q, dtype=np.float64)
    N, C = q.shape
    return (q.reshape(N, C // block, block) * np.asarray(s, dtype=np.float64)[..., None]).reshape(N, C)
