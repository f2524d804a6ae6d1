"""Lightning-indexer scores and top-k selection (test infrastructure).

Pages: "DeepSeek-V4", Design overview (CSA applies the lightning-indexer sparse
attention of V3.2 to the compressed entries) and Inference efficiency (the
indexer QK path); "Why DeepSeek V4 Stands Apart", Core Architectural
Innovations (top-1024 entries per query for Pro, top-512 for Flash).

Reading: the score of compressed entry j for one query is
    s_j = sum_r omega_r * max(0, p_r . key_j)
over the H_I indexer heads r, with one shared indexer key per entry, no scale
and no normalisation.  Only entries whose window ends at or before the query
position are candidates.  The k selected entries are the candidates of largest
score, ties broken toward the smaller entry index; when fewer than k entries
are visible, all of them are selected.
"""
import numpy as np


def scores(p, omega, keys):
    """p: [H_I, d_I], omega: [H_I], keys: [N, d_I] -> [N] float64."""
    p = np.asarray(p, dtype=np.float64)
    omega = np.asarray(omega, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros(0, dtype=np.float64)
    dots = keys @ p.T                      # [N, H_I]
    return np.maximum(dots, 0.0) @ omega   # [N]


def topk(s, k: int):
    """Indices of the k largest scores, ties -> smaller index, in rank order."""
    s = np.asarray(s, dtype=np.float64)
    j = np.arange(s.shape[0])
    order = np.lexsort((j, -s))            # primary: -s ascending, secondary: j
    return order[:min(k, s.shape[0])]


def kth_score(s, k: int):
    """Score of the last selected entry (None when every entry is selected)."""
    if s.shape[0] <= k:
        return None
    return float(s[topk(s, k)[-1]])
