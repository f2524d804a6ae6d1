"""Softmax attention pieces: partials, sink and merge (test infrastructure).

Pages: "DeepSeek-V4", Inference efficiency (one KV head shared by all query
heads), Core block and Provenance references 17-18 (RMSNorm on queries and on
compressed KV entries; attention sinks); "Why DeepSeek V4 Stands Apart", Core
Architectural Innovations (128-token sliding window; sparse attention over the
selected CSA entries; dense attention over the HCA entries).

Readings: a compressed entry serves as both key and value (K = V), unless
the layer takes its values from a separate raw stream (then every key row has
a value row beside it, built by the same steps);
logits are scale * qhat_h . key with scale = 1/sqrt(D); the sink of head h is
one logit sigma_h with a zero value, so it only enlarges the denominator.

A *partial* over a key subset P is (o_P, lse_P) with lse_P = log sum exp(l) and
o_P = sum softmax_P(l) * key; the empty set gives (0, -inf).  Partials over a
partition of the key set combine exactly: lse = log(sum exp(lse_p) + exp(sigma))
and o = sum exp(lse_p - lse) * o_p.
"""
import numpy as np

from .compress import rmsnorm
from .numerics import round_to
from .rope import BASE, rotate


def normalize_query(q, eps: float, dtype: str, pos=None, rope: int = 0, base: float = BASE):
    """q: [H, D] raw -> RMS-normalised per head (then, with rope > 0, turned
    by the query position pos on its last rope dims), rounded to the KV type."""
    qn = rmsnorm(q, eps)
    if rope:
        qn = rotate(qn, pos, rope, base)
    return round_to(qn, dtype)


def normalize_tokens(x, eps: float, dtype: str, pos=None, rope: int = 0, base: float = BASE):
    """Raw window tokens [n, D] -> RMS-normalised keys (with rope > 0, token
    r turned by its position pos[r]), rounded to the KV type."""
    xn = rmsnorm(x, eps)
    if rope:
        xn = rotate(xn, pos, rope, base)
    return round_to(xn, dtype)


def logits(qhat, keys, scale: float):
    """qhat [H, D], keys [n, D] -> [H, n]."""
    return scale * (np.asarray(qhat, np.float64) @ np.asarray(keys, np.float64).T)


def partial(qhat, keys, scale: float, values=None):
    """Normalised partial attention of every head over ``keys``, averaging
    ``values`` (row n the value of key n; None: the keys themselves).

    Returns o [H, D] and lse [H]; an empty key set gives o = 0, lse = -inf."""
    qhat = np.asarray(qhat, np.float64)
    keys = np.asarray(keys, np.float64)
    vals = keys if values is None else np.asarray(values, np.float64)
    if vals.shape != keys.shape:
        raise ValueError("one value row per key row")
    H, D = qhat.shape
    if keys.shape[0] == 0:
        return np.zeros((H, D)), np.full(H, -np.inf)
    lg = logits(qhat, keys, scale)                    # [H, n]
    mx = np.max(lg, axis=1, keepdims=True)
    e = np.exp(lg - mx)
    se = np.sum(e, axis=1, keepdims=True)
    o = (e / se) @ vals
    lse = (mx + np.log(se))[:, 0]
    return o, lse


def merge(parts, sigma=None):
    """Combine partials [(o [H, D], lse [H]), ...] and an optional sink [H].

    Returns (o [H, D], lse [H]) of the union, the sink counted in the
    denominator only."""
    H, D = parts[0][0].shape if parts else (len(sigma), 0)
    lses = [np.asarray(l, np.float64) for _, l in parts]
    if sigma is not None:
        lses.append(np.asarray(sigma, np.float64))
    stack = np.stack(lses, axis=0)                    # [P, H]
    mx = np.max(stack, axis=0)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    with np.errstate(divide="ignore"):                # all parts empty -> log(0) = -inf
        tot = safe + np.log(np.sum(np.exp(stack - safe), axis=0))
    tot = np.where(np.isfinite(mx), tot, -np.inf)
    o = np.zeros((H, D))
    for o_p, l_p in parts:
        wgt = np.where(np.isfinite(l_p), np.exp(np.asarray(l_p) - np.where(np.isfinite(tot), tot, 0.0)), 0.0)
        o = o + wgt[:, None] * np.asarray(o_p, np.float64)
    return o, tot


def attend(qhat, keys, scale: float, sigma=None, values=None):
    """One softmax over ``keys`` plus the sink, written directly (no partials).

    Returns o [H, D] and the per-head probabilities [H, n] and sink
    probability [H] (so callers can check that they sum to one)."""
    qhat = np.asarray(qhat, np.float64)
    keys = np.asarray(keys, np.float64)
    vals = keys if values is None else np.asarray(values, np.float64)
    lg = logits(qhat, keys, scale)
    cols = [lg]
    if sigma is not None:
        cols.append(np.asarray(sigma, np.float64)[:, None])
    allg = np.concatenate(cols, axis=1)
    mx = np.max(allg, axis=1, keepdims=True)
    e = np.exp(allg - mx)
    prob = e / np.sum(e, axis=1, keepdims=True)
    n = keys.shape[0]
    o = prob[:, :n] @ vals
    psink = prob[:, n] if sigma is not None else np.zeros(qhat.shape[0])
    return o, prob[:, :n], psink
