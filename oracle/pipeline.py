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

Options: the dual-stream compressor (cfg.dual: the CSA windows' second halves
from the streams x_b, a_b, u_b, c_b; see oracle.compress) and separate values
(cfg.sepv: a raw value stream v, pooled with the key entries' logits over the
same windows -- in the dual form its second halves from v_b -- and normalised
and turned as the keys; the window's values are the raw v tokens, normalised
and turned as the window keys).

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
from .rope import entry_positions, rotate


@dataclass
class SeqCaches:
    kv_csa: np.ndarray   # [N_csa, D]
    ikey: np.ndarray     # [N_csa, dI]
    kv_hca: np.ndarray   # [N_hca, D]
    v_csa: Optional[np.ndarray] = None   # value rows of the CSA entries (separate values), else None
    v_hca: Optional[np.ndarray] = None


def seq_slice(arr, tok_off, b):
    return np.asarray(arr[int(tok_off[b]):int(tok_off[b + 1])], dtype=np.float64)


def fp8_keys(cfg) -> bool:
    """Indexer keys stored as E4M3 rows with a scale (oracle.quant)."""
    return getattr(cfg, "ikey", "bf16") == "fp8"


def kv_entries(src, z, m, w, cfg, entries=None, src2=None, z2=None):
    """RMS-normalised KV entries of one stream (with cfg.rope, entry j turned
    by the position of its window's last token), rounded to the storage type;
    src2, z2: the second-half stream of the dual-stream form."""
    e = compress(src, z, m, w, True, cfg.eps, entries, src2=src2, z2=z2)
    rope = getattr(cfg, "rope", 0)
    if rope and len(e):
        js = range(n_entries(src.shape[0], m, w)) if entries is None else entries
        e = rotate(e, entry_positions(js, m, w), rope, cfg.rope_base)
    return round_to(e, cfg.dtype)


def build_seq_caches(x, a, g, u, c, cfg, opt=None) -> SeqCaches:
    """Caches of one sequence from its raw streams (all float64 views).  With
    fp8 or MXFP4 indexer keys the key cache holds the rows they stand for.
    opt: the option streams of the sequence (x_b, a_b, u_b, c_b with
    cfg.dual; v, and v_b with both options, with cfg.sepv)."""
    opt = opt or {}
    dual = getattr(cfg, "dual", False)
    sepv = getattr(cfg, "sepv", False)
    second = (lambda k: opt[k]) if dual else (lambda k: None)  # noqa: E731
    kv_csa = kv_entries(x, a, cfg.m, cfg.w, cfg, src2=second("x_b"), z2=second("a_b"))
    pooled = compress(u, c, cfg.m, cfg.w, False, cfg.eps, src2=second("u_b"), z2=second("c_b"))
    kind = getattr(cfg, "ikey", "bf16")
    if kind == "fp8":
        ikey = quant.dequantize_rows(*quant.quantize_rows(pooled))
    elif kind == "mxfp4":
        ikey = quant.dequantize_mx_rows(*quant.quantize_mx_rows(pooled))
    else:
        ikey = round_to(pooled, cfg.dtype)
    kv_hca = kv_entries(x, g, cfg.m2, cfg.w2, cfg)
    v_csa = v_hca = None
    if sepv:
        v_csa = kv_entries(opt["v"], a, cfg.m, cfg.w, cfg, src2=second("v_b"), z2=second("a_b"))
        v_hca = kv_entries(opt["v"], g, cfg.m2, cfg.w2, cfg)
    return SeqCaches(kv_csa, ikey, kv_hca, v_csa, v_hca)


OPTION_STREAMS = ("x_b", "a_b", "u_b", "c_b", "v", "v_b")


def build_caches(raw, cfg) -> List[SeqCaches]:
    off = raw["tok_off"]
    out = []
    for b in range(cfg.B):
        s = lambda k: seq_slice(raw[k], off, b)  # noqa: E731
        opt = {k: s(k) for k in OPTION_STREAMS if k in raw}
        out.append(build_seq_caches(s("x"), s("a"), s("g"), s("u"), s("c"), cfg, opt))
    return out


def select(ikey, p, omega, i, cfg):
    """Visible CSA entries, their scores and the selected indices for query i
    (with fp8 indexer keys, ikey holds the rows they stand for)."""
    nv = n_visible(i, cfg.m, cfg.w)
    s = scores(p, omega, ikey[:nv])
    return s, topk(s, cfg.k)


def window_keys(x_seq, i, cfg):
    lo = max(0, i - cfg.W + 1)
    return att.normalize_tokens(x_seq[lo:i + 1], cfg.eps, cfg.dtype, pos=np.arange(lo, i + 1),
                                rope=getattr(cfg, "rope", 0), base=getattr(cfg, "rope_base", 10000.0))


def finish(o, i, cfg):
    """The attention output of the query at position i: with cfg.rope turned
    by -i (the values carry their own positions' rotation), then rounded."""
    rope = getattr(cfg, "rope", 0)
    if rope:
        o = rotate(o, -i, rope, cfg.rope_base)
    return round_to(o, cfg.dtype)


def query_step(caches: SeqCaches, x_seq, q, p, omega, sigma, i, cfg, idx=None, v_seq=None):
    """Every intermediate of one query (float64; outputs rounded at the end).

    ``idx`` overrides the selection (to attend over another selected set);
    ``v_seq``: the sequence's raw value tokens (separate values)."""
    s, sel = select(caches.ikey, p, omega, i, cfg)
    if idx is None:
        idx = sel
    qhat = att.normalize_query(q, cfg.eps, cfg.dtype, pos=i, rope=getattr(cfg, "rope", 0),
                               base=getattr(cfg, "rope_base", 10000.0))
    idx = np.asarray(idx, dtype=np.int64)
    idx = idx[idx >= 0]
    sepv = getattr(cfg, "sepv", False)
    if sepv and (caches.v_csa is None or v_seq is None):
        raise ValueError("separate values need the value caches and the raw value tokens")
    csa = att.partial(qhat, caches.kv_csa[idx], cfg.scale, caches.v_csa[idx] if sepv else None)
    nh = n_visible(i, cfg.m2, cfg.w2)
    hca = att.partial(qhat, caches.kv_hca[:nh], cfg.scale, caches.v_hca[:nh] if sepv else None)
    swa = att.partial(qhat, window_keys(x_seq, i, cfg), cfg.scale, window_keys(v_seq, i, cfg) if sepv else None)
    o_a, lse_a = att.merge([csa, hca, swa], sigma)
    o_csa, _ = att.merge([csa, swa], sigma)
    o_hca, _ = att.merge([hca, swa], sigma)
    return dict(scores=s, sel=sel, idx=idx, qhat=qhat, csa=csa, hca=hca, swa=swa,
                out=finish(o_a, i, cfg), out_raw=o_a, lse=lse_a,
                out_csa=finish(o_csa, i, cfg), out_hca=finish(o_hca, i, cfg))


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
                                 raw["omega"][r], raw["sigma"], i, cfg,
                                 v_seq=seq_slice(raw["v"], off, b) if getattr(cfg, "sepv", False) else None)
    return caches, res


__all__ = ["SeqCaches", "kv_entries", "build_seq_caches", "build_caches", "select", "window_keys", "finish",
           "query_step", "run", "n_entries", "n_visible"]
