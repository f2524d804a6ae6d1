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
