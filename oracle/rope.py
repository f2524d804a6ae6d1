"""Partial rotary position embedding (test infrastructure; see oracle/__init__).

Pages: "DeepSeek-V4" spec sheet, Core block (partial RoPE: yes) and
Provenance 16 (RoPE on the last 64 dims, with a -i RoPE on the outputs).  The
pages give nothing more; the readings taken:

* The rotation is the rotary embedding in its original complex form: the
  rotated dims are taken in consecutive pairs (2p, 2p+1), each pair read as
  the complex number x[2p] + i x[2p+1] and multiplied by exp(i pos theta_p)
  with theta_p = base ** (-2p / d_rope) and base = 10000 (the textbook value;
  the pages name no base and no context-length scaling, so none is applied).
* The rotated dims are the last d_rope = 64 of a head (every dim when
  D <= 64); the first D - d_rope dims are not rotated.
* Positions: the query at position i turns by i; a raw window token at t by
  t; a compressed entry by the position of the last token of its window,
  j*m + w - 1 (the position from which it is visible).
* Order: RMSNorm, then the rotation (it keeps each pair's length, so the RMS
  is the same before and after), then rounding to the storage type.
  Compressed entries are stored rotated; since an entry is both key and
  value, the attention output carries the rotations of the values it
  averages, and it is turned by -i (the "-i RoPE on outputs"), so that every
  value enters at its position relative to the query.
* The lightning indexer's queries and keys are not rotated.
"""
import numpy as np

BASE = 10000.0


def rotate(x, pos, d_rope: int, base: float = BASE):
    """x [..., D] turned by the angles of position(s) pos (a scalar, or an
    array broadcasting against x[..., 0]) on its last min(d_rope, D) dims."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    dr = min(int(d_rope), D)
    if dr <= 0:
        return x.copy()
    if dr % 2:
        raise ValueError("d_rope must be even")
    p = np.arange(dr // 2, dtype=np.float64)
    theta = base ** (-2.0 * p / dr)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    lo = D - dr
    z = (x[..., lo::2] + 1j * x[..., lo + 1::2]) * np.exp(1j * ang)
    out = x.copy()
    out[..., lo::2] = z.real
    out[..., lo + 1::2] = z.imag
    return out


def entry_positions(entries, m: int, w: int):
    """Position of compressed entry j: the last token of its window."""
    return np.asarray(list(entries), dtype=np.int64) * m + (w - 1)
