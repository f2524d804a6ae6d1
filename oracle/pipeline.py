"""The decode / prefill step composed from the oracle pieces (test infrastructure).

One query token of sequence b at position i (decode: i = L_b - 1, the query
token is already part of the context; prefill: every position of the chunk):

1. compress the raw streams into the CSA KV cache (m=4, w=8, RMSNorm), the CSA
   indexer-key cache (m=4, w=8, no norm) and the HCA cache (m=w=128, RMSNorm),
   each rounded to the storage type;
2. score the visible CSA entries with the lightning indexer, keep the top k;
3. attend with the RMS-normalised query over
     - the k selected CSA entries                          (csa partial)
     - every visible HCA entry                             (hca partial)
     - the raw tokens max(0, i-W+1) .. i, RMS-normalised   (swa partial)
   and the sink, merged into one softmax ("mode A", one layer holding all
   three branches), or as two layer outputs ("mode B": CSA + window + sink and
   HCA + window + sink).

Pages: "Why DeepSeek V4 Stands Apart", Core Architectural Innovations; "DeepSeek-V4",
Design overview, Core block, Inference efficiency; "DeepSeek V4 Is Not a Better
Model", 1. CSA + HCA (older tokens compressed, recent tokens kept at full
resolution).  The readings taken are stated in the modules this one calls.
"""
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from . import attention as att
from .compress import compress, n_entries, n_visible
from . import quant
from .indexer import scores, topk
from .numerics import round_to


@dataclass
class SeqCaches:
    kv_csa: np.ndarray   # [N_csa, D]
    ikey: np.ndarray     # [N_csa, dI]
    kv_hca: np.ndarray   # [N_hca, D]


def seq_slice(arr, tok_off, b):
    return np.asarray(arr[int(tok_off[b]):int(tok_off[b + 1])], dtype=np.float64)


def fp8_keys(cfg) -> bool:
    """Indexer keys stored as E4M3 rows with a scale (oracle.quant)."""
    return getattr(cfg, "ikey", "bf16") == "fp8"


def build_seq_caches(x, a, g, u, c, cfg) -> SeqCaches:
    """Caches of one sequence from its raw streams (all float64 views).  With
    fp8 or MXFP4 indexer keys the key cache holds the rows they stand for."""
    kv_csa = round_to(compress(x, a, cfg.m, cfg.w, True, cfg.eps), cfg.dtype)
    pooled = compress(u, c, cfg.m, cfg.w, False, cfg.eps)
    kind = getattr(cfg, "ikey", "bf16")
    if kind == "fp8":
        ikey = quant.dequantize_rows(*quant.quantize_rows(pooled))
    elif kind == "mxfp4":
        ikey = quant.dequantize_mx_rows(*quant.quantize_mx_rows(pooled))
    else:
        ikey = round_to(pooled, cfg.dtype)
    kv_hca = round_to(compress(x, g, cfg.m2, cfg.w2, True, cfg.eps), cfg.dtype)
    return SeqCaches(kv_csa, ikey, kv_hca)


def build_caches(raw, cfg) -> List[SeqCaches]:
    off = raw["tok_off"]
    out = []
    for b in range(cfg.B):
        s = lambda k: seq_slice(raw[k], off, b)  # noqa: E731
        out.append(build_seq_caches(s("x"), s("a"), s("g"), s("u"), s("c"), cfg))
    return out


def select(ikey, p, omega, i, cfg):
    """Visible CSA entries, their scores and the selected indices for query i
    (with fp8 indexer keys, ikey holds the rows they stand for)."""
    nv = n_visible(i, cfg.m, cfg.w)
    s = scores(p, omega, ikey[:nv])
    return s, topk(s, cfg.k)


def window_keys(x_seq, i, cfg):
    lo = max(0, i - cfg.W + 1)
    return att.normalize_tokens(x_seq[lo:i + 1], cfg.eps, cfg.dtype)


def query_step(caches: SeqCaches, x_seq, q, p, omega, sigma, i, cfg, idx=None):
    """Every intermediate of one query (float64; outputs rounded at the end).

    ``idx`` overrides the selection (to attend over another selected set)."""
    s, sel = select(caches.ikey, p, omega, i, cfg)
    if idx is None:
        idx = sel
    qhat = att.normalize_query(q, cfg.eps, cfg.dtype)
    idx = np.asarray(idx, dtype=np.int64)
    idx = idx[idx >= 0]
    csa = att.partial(qhat, caches.kv_csa[idx], cfg.scale)
    nh = n_visible(i, cfg.m2, cfg.w2)
    hca = att.partial(qhat, caches.kv_hca[:nh], cfg.scale)
    swa = att.partial(qhat, window_keys(x_seq, i, cfg), cfg.scale)
    o_a, lse_a = att.merge([csa, hca, swa], sigma)
    o_csa, _ = att.merge([csa, swa], sigma)
    o_hca, _ = att.merge([hca, swa], sigma)
    return dict(scores=s, sel=sel, idx=idx, qhat=qhat, csa=csa, hca=hca, swa=swa,
                out=round_to(o_a, cfg.dtype), out_raw=o_a, lse=lse_a,
                out_csa=round_to(o_csa, cfg.dtype), out_hca=round_to(o_hca, cfg.dtype))


def run(raw, cfg, caches: Optional[List[SeqCaches]] = None, queries=None):
    """All queries of a workload: returns (caches, {(b, t): query_step dict}).

    ``queries`` optionally restricts to a list of (b, t) pairs, t indexing the
    cfg.tq query tokens of sequence b."""
    if caches is None:
        caches = build_caches(raw, cfg)
    off = raw["tok_off"]
    res = {}
    if queries is None:
        queries = [(b, t) for b in range(cfg.B) for t in range(cfg.tq)]
    for b, t in queries:
        r = b * cfg.tq + t
        i = int(raw["q_pos"][b, t])
        res[(b, t)] = query_step(caches[b], seq_slice(raw["x"], off, b), raw["q"][r], raw["p"][r],
                                 raw["omega"][r], raw["sigma"], i, cfg)
    return caches, res


__all__ = ["SeqCaches", "build_seq_caches", "build_caches", "select", "window_keys",
           "query_step", "run", "n_entries", "n_visible"]
