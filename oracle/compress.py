"""KV compression (test infrastructure; see oracle/__init__).

Pages: "Why DeepSeek V4 Stands Apart", Core Architectural Innovations (CSA
compresses KV entries 4x; HCA compresses 128:1); "DeepSeek-V4", Design overview
(CSA compresses every 4 tokens into two overlapping streams; HCA uses m'=128)
and Provenance reference 17 (RMSNorm on the compressed KV entries).

Readings: entry j of a stream with stride m and window w pools the
tokens t = j*m .. j*m+w-1 with weights softmax_t(z[t, c]) taken separately for
every channel c; only complete windows exist, so a sequence of L tokens has
N(L) = 0 if L < w else (L - w) // m + 1 entries.  CSA uses m=4, w=8 (each token
feeds two consecutive windows: the "two overlapping streams"), HCA uses
m = w = 128.  KV entries are then RMS-normalised over channels with unit gain:
e / sqrt(mean(e**2) + eps).  Indexer keys are pooled the same way (CSA windows)
but not normalised.

Dual-stream form (the other reading of "two overlapping streams"; CSA only,
w = 2m): every token t carries two (value, logit) pairs, one for the window
in whose first half it lies (window t // m: src, z) and one for the window in
whose second half it lies (window t // m - 1: src2, z2).  An entry pools its
first m tokens from the first pair and its last m tokens from the second,
under one softmax over all w logits of a channel.
"""
import numpy as np


def n_entries(L: int, m: int, w: int) -> int:
    """Number of complete windows of length w at stride m in L tokens."""
    if L < w:
        return 0
    return (L - w) // m + 1


def n_visible(i: int, m: int, w: int) -> int:
    """Entries whose whole window lies at or before query position i."""
    return n_entries(i + 1, m, w)


def rmsnorm(v, eps: float):
    """RMSNorm with unit gain over the last axis."""
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps)


def pool_window(src_win, z_win):
    """Softmax-weighted pool of one window.

    src_win: [w, C]; z_win: [w, C] per-channel logits or [w] per-token logits.
    Returns ([C] pooled vector, [w, C] weights)."""
    src_win = np.asarray(src_win, dtype=np.float64)
    z = np.asarray(z_win, dtype=np.float64)
    if z.ndim == 1:
        z = np.repeat(z[:, None], src_win.shape[1], axis=1)
    zmax = np.max(z, axis=0, keepdims=True)
    ez = np.exp(z - zmax)
    alpha = ez / np.sum(ez, axis=0, keepdims=True)
    return np.sum(alpha * src_win, axis=0), alpha


def compress(src, z, m: int, w: int, norm: bool, eps: float = 1e-6, entries=None, src2=None, z2=None):
    """Compressed entries of one sequence (float64, not yet rounded).

    src: [L, C] raw stream of the sequence; z: [L, C] or [L] pooling logits.
    entries: optional iterable of entry indices to compute (default: all).
    src2, z2: the second-half stream of the dual-stream form (w = 2m), or
    None.  Returns [len(entries), C]."""
    L = src.shape[0]
    N = n_entries(L, m, w)
    dual = src2 is not None
    if dual and (w != 2 * m or z2 is None or np.shape(src2) != np.shape(src) or np.shape(z2) != np.shape(z)):
        raise ValueError("the dual-stream form needs w = 2m and second-half streams shaped as the first")
    if entries is None:
        entries = range(N)
    entries = list(entries)
    C = src.shape[1]
    out = np.zeros((len(entries), C), dtype=np.float64)
    for r, j in enumerate(entries):
        if not (0 <= j < N):
            raise IndexError(f"entry {j} outside [0, {N})")
        t0 = j * m
        if dual:
            # the window's rows: its first half from the first stream, its
            # second half from the second
            xs = np.concatenate([np.asarray(src[t0:t0 + m]), np.asarray(src2[t0 + m:t0 + w])])
            zs = np.concatenate([np.asarray(z[t0:t0 + m]), np.asarray(z2[t0 + m:t0 + w])])
            e, _ = pool_window(xs, zs)
        else:
            e, _ = pool_window(src[t0:t0 + w], z[t0:t0 + w])
        out[r] = e
    if norm and len(entries):
        out = rmsnorm(out, eps)
    return out
