#!/usr/bin/env python3
"""Decode throughput of one hybrid compressed attention layer on one MI355X.

Metric: decode query-tokens/s per layer at a 1M-token Pro-shaped context, and
the fraction of peak HBM bandwidth it corresponds to.

A step is one pass of the whole hot path for one query token per sequence:
  csa_index_score_append (the CSA, indexer-key and HCA entries the new token
    completes, and the index scores, in one launch)
  -> hybrid_attn (one launch: the sparse blocks filter the scores and each
    selects its share of the exact top-k; CSA sparse + HCA dense + window
    partials)
  -> swa_merge (sink + merge)
on one stream, over caches resident in HBM.  To keep the 256 MB Infinity Cache from serving
the caches, steps rotate over R layers, each with its own raw streams and
caches (R * per-step bytes >= 2 x 256 MB).

Timed regions (HIP events on the launch stream, synchronised on both sides):
  1. per kernel: one HIP graph of that kernel's launch for each of the R
     rotated layers, replayed 8 times (the attention launch, which selects
     from what the score kernel leaves in the index workspace, is timed
     after it, the score kernel's time subtracted); the dominant kernel's
     average launch duration gives the roofline;
  2. the headline: the W warmup steps and then the K timed steps, each set
     captured as one HIP graph of consecutive layer steps and replayed once.
     With one sequence the K steps are K consecutive decode positions, each
     appending what its token completes (so appends are amortized as they
     occur); also reported: the step at the last position, where the token
     completes a CSA, an indexer and an HCA entry at once;
  3. the same K steps launched directly (host launch cost included).
cpu_baseline: the float64 oracle on the host, same workload, bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X

# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE and, in a run
# of its own, WRITE_SIZE on this benchmark (the summary and the commands are
# in profiles/hbm_traffic_pro_1m_decode.md), each scaled by what the counter
# reads for a plain 256 MiB device copy (FETCH_SIZE reports half the bytes the
# copy reads: x2; WRITE_SIZE all it writes: x1).  A figure holds for the
# kernel source it was taken on: the SHA-1 of the files the kernel is built
# from; any change makes the reported traffic null until it is measured again.
TRAFFIC = {
    ("pro_1m_decode", "hybrid_attn"): {
        "files": ["long_context_attention_20_amd/csrc/lca_attention.hip",
                  "long_context_attention_20_amd/csrc/lca_attn_block.h",
                  "long_context_attention_20_amd/csrc/lca_common.h",
                  "long_context_attention_20_amd/csrc/lca_topk.h"],
        "sha1": "e362f2287aa9db536844baaae2d523b5d404c0bc",
        "fetch_kib": 6388.1, "write_kib": 9013.3, "fetch_scale": 2.0, "write_scale": 1.0,
    },
}


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the counter runs, or None when
    none was taken on the current source."""
    import hashlib
    t = TRAFFIC.get((workload, kernel))
    if t is None:
        return None
    h = hashlib.sha1()
    for f in t["files"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != t["sha1"]:
        return None
    return (t["fetch_kib"] * t["fetch_scale"] + t["write_kib"] * t["write_scale"]) * 1024
MFMA_BF16_PEAK = 2.5e15    # dense bf16 FLOP/s, MI355X
MALL_BYTES = 256 << 20
MTP_MAX_ROWS = 4           # query rows per sequence timed as a decode step (more: a prefill chunk)


def n_windows(L, m, w):
    return 0 if L < w else (L - w) // m + 1


def key_bytes(cfg):
    """Bytes of one indexer key in the cache: d_I elements, or for fp8 rows
    d_I E4M3 bytes + the fp32 scale + 4 pad bytes."""
    if cfg.ikey == "fp8":
        return cfg.dI + 8
    if cfg.ikey == "mxfp4":
        return cfg.dI // 2 + 8
    return cfg.dI * (2 if cfg.dtype == "bf16" else 4)


def step_bytes(cfg):
    """Algorithmic HBM bytes of one decode step: what the method must move.
    With tq query rows per sequence the indexer keys, the HCA entries and the
    window rows are read once for all of them; each row has its own
    selection, query and output."""
    e = 2 if cfg.dtype == "bf16" else 4
    tq = cfg.tq
    tot = 0
    for L in cfg.lens:
        ncsa = n_windows(L, cfg.m, cfg.w)
        nh = n_windows(L, cfg.m2, cfg.w2)
        kk = min(cfg.k, ncsa)
        kv = 2 if cfg.sepv else 1                       # key rows, and value rows beside them
        tot += ncsa * key_bytes(cfg)                    # indexer keys
        tot += tq * kk * (kv * cfg.D * e + 4)           # selected entries + indices, per row
        tot += kv * min(cfg.W + tq - 1, L) * cfg.D * e  # window rows
        tot += kv * nh * cfg.D * e                      # HCA entries
        tot += tq * (cfg.H * cfg.D * 2 * e + cfg.H * 4)  # q, out, sink per row
    return tot


METRIC = "decode query-tokens/s per layer at 1M ctx (Pro shape); % of HBM peak BW"


def metric_name(cfg):
    """The headline metric for the Pro 1M decode; for other workloads the
    same measure, named with what differs."""
    if cfg.name == "pro_1m_decode":
        return METRIC
    what = []
    if cfg.ikey != "bf16":
        what.append(f"{cfg.ikey} indexer keys")
    if cfg.tq > 1:
        what.append(f"{cfg.tq} query rows per step: the main token and {cfg.tq - 1} drafted")
    if cfg.rope:
        what.append(f"rotary embedding on {cfg.rope} dims")
    if cfg.dual:
        what.append("dual-stream compressor")
    if cfg.sepv:
        what.append("separate values")
    if cfg.name.startswith("pro_1m"):
        where = "1M ctx (Pro shape" + "".join(", " + w for w in what) + ")"
    else:
        where = f"the {cfg.name} workload" + (" (" + ", ".join(what) + ")" if what else "")
    return f"decode query-tokens/s per layer at {where}; % of HBM peak BW"


def kernel_cost(cfg, name, front=False):
    """(bytes, flops, overhead bytes) of one launch of a step's kernel: the
    bytes are its share of the step's algorithmic bytes (the byte model of
    step_bytes: keys shared by the tq rows of a sequence counted once); the
    overhead is traffic the design adds that the method does not need (the
    row's scores written by the scoring launch and read back by the sparse
    blocks).  front: the step in front form, where the HCA entries and the
    window are attended beside the scores rather than in hybrid_attn."""
    e = 2 if cfg.dtype == "bf16" else 4
    tq = cfg.tq
    kv = 2 if cfg.sepv else 1                                    # key rows, and value rows beside them
    by = fl = ov = 0
    for L in cfg.lens:
        ncsa = n_windows(L, cfg.m, cfg.w)
        nh = n_windows(L, cfg.m2, cfg.w2)
        kk = min(cfg.k, ncsa)
        nwin = min(cfg.W + tq - 1, L)
        if name in ("csa_index_score", "csa_index_score_append", "decode_front"):
            by += ncsa * key_bytes(cfg)
            fl += 2 * ncsa * cfg.dI * cfg.HI * tq
            ov += tq * ncsa * 4                                  # scores written
        if name in ("csa_index_score_append", "decode_front"):  # the entries the new tokens complete
            by += (kv * (2 * cfg.w * cfg.D + 2 * cfg.w2 * cfg.D) + 2 * cfg.w * cfg.dI) * e + (kv * 2 * cfg.D + cfg.dI) * e
        if name == "decode_front":                               # HCA entries, window rows, the queries
            by += kv * (nh + nwin) * cfg.D * e + tq * cfg.H * cfg.D * e
            fl += 4 * cfg.H * cfg.D * (nh + min(cfg.W, L)) * tq
        if name == "csa_topk_select":
            by += kk * 4
            ov += tq * ncsa * 4
        if name == "csa_sparse_attn":
            by += kk * cfg.D * e + cfg.H * cfg.D * e
            fl += 4 * cfg.H * cfg.D * kk
        if name == "hca_attn":
            by += nh * cfg.D * e + cfg.H * cfg.D * e
            fl += 4 * cfg.H * cfg.D * nh
        if name == "swa_attn":
            by += min(cfg.W, L) * cfg.D * e + cfg.H * cfg.D * e
            fl += 4 * cfg.H * cfg.D * min(cfg.W, L)
        if name == "hybrid_attn":                                # the selection + the sparse branch
            by += tq * kk * (kv * cfg.D * e + 4) + tq * cfg.H * cfg.D * e
            fl += 4 * cfg.H * cfg.D * kk * tq
            ov += tq * ncsa * 4                                  # the row's scores read back
            if not front:                                        # the HCA entries and the window
                by += kv * (nh + nwin) * cfg.D * e
                fl += 4 * cfg.H * cfg.D * (nh + min(cfg.W, L)) * tq
        if name == "swa_merge":
            by += tq * (cfg.H * cfg.D * e + cfg.H * 4)           # output + sink
    return by, fl, ov


class LayerState:
    """One layer's inputs and caches, all resident on the GPU."""

    def __init__(self, cfg, layer, attn, dev):
        import torch
        import lca_inputs as li
        raw = li.make_raw_torch(cfg, layer, dev)
        self.raw = raw
        self.caches = attn.alloc_caches(cfg.lens, dev, raw["x"].dtype)
        attn.compress(self.caches, raw, raw["tok_off"])                     # cache build
        self.q, self.p, self.omega, self.sigma = raw["q"], raw["p"], raw["omega"], raw["sigma"]
        self.q_pos = raw["q_pos"].reshape(-1).contiguous()
        self.tok_off = raw["tok_off"]
        self.done_h = [L - cfg.tq for L in cfg.lens]
        self.done = torch.tensor(self.done_h, dtype=torch.int64, device=dev)


class Position:
    """A decode step of a one-sequence workload ending at token position p:
    the sequence is read as its first p + 1 tokens and the step's tq query
    rows sit at positions p - tq + 1 .. p, so the step appends exactly the
    entries those tokens complete."""

    def __init__(self, p, dev, tq=1):
        import torch
        self.p = p
        self.tok_off = torch.tensor([0, p + 1], dtype=torch.int64, device=dev)
        self.q_pos = torch.arange(p - tq + 1, p + 1, dtype=torch.int32, device=dev)
        self.done = torch.tensor([p + 1 - tq], dtype=torch.int64, device=dev)
        self.done_h = [p + 1 - tq]
        self.lens_h = [p + 1]


class Runner:
    def __init__(self, cfg, R, dev, split_csa=0, split_hca=0, front=None, half_partials=True, batch_invariant=False):
        import torch
        from long_context_attention_20_amd import HybridAttention, ops
        self.torch, self.ops = torch, ops
        self.cfg = cfg
        a = HybridAttention(cfg.H, cfg.D, cfg.HI, cfg.dI, cfg.k, cfg.m, cfg.w, cfg.m2, cfg.w2, cfg.W, cfg.eps,
                            split_csa=split_csa or None, split_hca=split_hca or None, ikey=cfg.ikey,
                            rope=cfg.rope, rope_base=cfg.rope_base, dual=cfg.dual, sepv=cfg.sepv,
                            half_partials=half_partials, batch_invariant=batch_invariant,
                            max_context=max(cfg.lens))
        self.attn = a
        self.layers = [LayerState(cfg, r, a, dev) for r in range(R)]
        rows = cfg.B * cfg.tq
        qmax = max(cfg.lens)
        self.bufs = a.decode_buffers(rows, n_windows(qmax, cfg.m, cfg.w), n_windows(qmax, cfg.m2, cfg.w2), dev,
                                     self.layers[0].q.dtype, front=front)
        self.front = self.bufs["front"]
        self.sc, self.sh, self.sw = self.bufs["sc"], self.bufs["sh"], self.bufs["sw"]
        first = "decode_front" if self.front else "csa_index_score_append"
        self.names = [first, "hybrid_attn", "swa_merge"]
        self.launches = {}  # kernels per call (default 1)
        # the attention launch selects from what the score launch leaves in
        # the index workspace (and clears it): it is timed after the score
        # launch, whose time is subtracted
        self.timed = [first, first + "+hybrid_attn", "swa_merge"]

    def step(self, L, pos=None):
        """The whole decode step (three calls on the current stream), at the
        last position of every sequence or at `pos` (one sequence)."""
        if pos is None:
            return self.attn.decode_step(L.caches, L.raw, L.tok_off, L.q, L.p, L.omega, L.sigma, L.q_pos, self.bufs,
                                         done_len=L.done, done_h=L.done_h)
        return self.attn.decode_step(L.caches, L.raw, pos.tok_off, L.q, L.p, L.omega, L.sigma, pos.q_pos, self.bufs,
                                     done_len=pos.done, done_h=pos.done_h, lens_h=pos.lens_h)

    def calls(self, L):
        """The same step (at the last position: every append) as its three
        single-kernel calls."""
        if self.front:
            return self.attn.front_calls(L.caches, L.raw, L.tok_off, L.q, L.p, L.omega, L.sigma, L.q_pos, self.bufs,
                                         L.done, L.done_h)
        cfg, ops, a, c, bf = self.cfg, self.ops, self.attn, L.caches, self.bufs
        st = a.compress_streams(c, L.raw, L.done_h)
        idx_st = [x for x in st if x["out"] is c.ikey][0]
        kv_st = [x for x in st if x["out"] is not c.ikey]
        srcs = a.attn_sources(c, L.raw["x"], L.tok_off, None, bf, L.raw.get("v"))
        parts = [bf["csa"], bf["hca"], bf["swa"]][:len(srcs)]
        return [
            lambda: ops.csa_index_score_append(L.p, L.omega, c.ikey, c.csa_off, L.q_pos, cfg.k, cfg.m, cfg.w,
                                               bf["max_csa"], bf["ws_idx"], idx_st, kv_st, L.tok_off, L.done,
                                               cfg.eps),
            lambda: ops.hybrid_attn(L.q, L.q_pos, srcs, a.scale, cfg.eps),
            lambda: ops.swa_merge(L.q, None, None, None, L.sigma, parts, 0, a.scale, cfg.eps, None, out=bf["out"]),
        ]

    def timed_call(self, L, name):
        """The call (or pair of calls) timed as `name`."""
        fs = dict(zip(self.names, self.calls(L)))
        parts = [fs[n] for n in name.split("+")]
        return lambda: [f() for f in parts]

    def step_calls(self, L):
        for f in self.calls(L):
            f()


def prefill_flops(cfg):
    """Algorithmic FLOPs of one prefill chunk step: indexer, sparse, HCA and
    window attention of every query row (2 FLOP per multiply-add)."""
    out = dict(indexer=0, sparse=0, hca=0, window=0)
    for b, L in enumerate(cfg.lens):
        for i in range(L - cfg.tq, L):
            nv = n_windows(i + 1, cfg.m, cfg.w)
            out["indexer"] += 2 * nv * cfg.dI * cfg.HI
            out["sparse"] += 4 * cfg.H * cfg.D * min(cfg.k, nv)
            out["hca"] += 4 * cfg.H * cfg.D * n_windows(i + 1, cfg.m2, cfg.w2)
            out["window"] += 4 * cfg.H * cfg.D * min(cfg.W, i + 1)
    return out


def run_prefill(cfg, args, dev):
    """One prefill chunk step per iteration: compress the chunk's entries,
    score and select for every query row, then attend and merge with the sink
    (one launch: every block takes the three branches for its rows and writes
    the output).  Reported against the matrix-core peak."""
    import torch
    import lca_inputs as li
    from long_context_attention_20_amd import HybridAttention, ops
    a = HybridAttention(cfg.H, cfg.D, cfg.HI, cfg.dI, cfg.k, cfg.m, cfg.w, cfg.m2, cfg.w2, cfg.W, cfg.eps,
                        ikey=cfg.ikey, rope=cfg.rope, rope_base=cfg.rope_base, dual=cfg.dual, sepv=cfg.sepv)
    raw = li.make_raw_torch(cfg, 0, dev)
    caches = a.alloc_caches(cfg.lens, dev, raw["x"].dtype)
    a.compress(caches, raw, raw["tok_off"])
    done_h = [L - cfg.tq for L in cfg.lens]
    done = torch.tensor(done_h, dtype=torch.int64, device=dev)
    q_pos = raw["q_pos"].reshape(-1).contiguous()
    q_pos_h = raw["q_pos"].reshape(-1).cpu().numpy()
    rows = q_pos.numel()
    qmax = int(q_pos_h.max()) + 1
    max_csa = n_windows(qmax, cfg.m, cfg.w)
    max_hca = n_windows(qmax, cfg.m2, cfg.w2)
    ws = a.index_workspace(rows, max_csa, dev)
    sc, sh, sw = a.fused_splits(rows, min(cfg.k, max_csa), max_hca, cfg.W)
    bufs = dict(sc=sc, sh=sh, sw=sw, max_hca=max_hca, csa=(None, None), hca=(None, None), swa=(None, None))
    idx = torch.empty((rows, cfg.k), dtype=torch.int32, device=dev)
    out = torch.empty_like(raw["q"])
    streams = a.compress_streams(caches, raw, done_h)
    # csa_index_topk with no scores requested: scores and selection in one
    # launch, no score stored
    names = ["kv_compress", "csa_index_topk", "hybrid_attn_merge"]
    srcs = a.attn_sources(caches, raw["x"], raw["tok_off"], idx, bufs, raw.get("v"))
    calls = [
        lambda: ops.kv_compress(streams, raw["tok_off"], done, cfg.eps),
        lambda: ops.csa_index_topk(raw["p"], raw["omega"], caches.ikey, caches.csa_off, q_pos, cfg.k, cfg.m, cfg.w,
                                   max_csa, ws, idx=idx),
        lambda: ops.hybrid_attn_merge(raw["q"], q_pos, srcs, raw["sigma"], a.scale, cfg.eps, out=out),
    ]
    K, W = max(1, min(args.steps, 10)), max(1, min(args.warmup, 2))
    for _ in range(W):
        for f in calls:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(K)]
    for it in range(K):
        ev[it][0].record()
        for j, f in enumerate(calls):
            f()
            ev[it][j + 1].record()
    torch.cuda.synchronize()
    per = np.array([[ev[it][j].elapsed_time(ev[it][j + 1]) for j in range(len(calls))] for it in range(K)]).mean(0)
    ms = float(per.sum())
    fl = prefill_flops(cfg)
    tot = sum(fl.values())
    j = names.index("hybrid_attn_merge")
    attn_fl = fl["sparse"] + fl["hca"] + fl["window"]
    res = {
        "metric": "prefill query-tokens/s per layer (Flash shape, 4096-token chunk after 256K); MFMA utilisation",
        "value": cfg.B * cfg.tq / (ms / 1e3),
        "unit": "q-tok/s/layer",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic (seeded N(0,1), generated on the GPU)",
        "config": {"workload": cfg.name, "cached": done_h[0], "chunk": cfg.tq, "q_heads": cfg.H, "head_dim": cfg.D,
                   "indexer": f"{cfg.HI}x{cfg.dI}", "topk": cfg.k, "splits": [sc, sh, sw],
                   "timing": "stream, events between the calls"},
        "flops_per_step": fl,
        "mfma_frac_of_peak": tot / (ms / 1e3) / MFMA_BF16_PEAK,
        "kernel_ms": {n: float(t) for n, t in zip(names, per)},
        "roofline": {"bound": "mfma", "kernel": "hybrid_attn_merge", "achieved": attn_fl / (per[j] / 1e3) / 1e12,
                     "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s",
                     "frac": attn_fl / (per[j] / 1e3) / MFMA_BF16_PEAK, "traffic": None,
                     "kernel_ms": float(per[j]), "flops_per_launch": attn_fl},
        "cpu_baseline": cpu_baseline_prefill(cfg, raw, args.cpu_seconds) if args.cpu_seconds > 0 else None,
    }
    print(json.dumps(res))


TRACE_PHASES = ["start", "filter done", "wait done", "selection done", "prologue done", "key loop done", "stored"]
KIND_NAMES = {0: "HCA (dense)", 1: "sparse (gather)", 2: "window", 3: "sparse (top-k inside)"}
SUB_PHASES = [(15, "filter loads issued"), (8, "histogram summed"), (9, "threshold found"), (10, "list space reserved"),
              (11, "own share counted"), (12, "lists loaded"), (13, "second threshold"), (14, "cut found")]


def trace_attention(run, path, reps=6):
    """Per-block phase stamps of the attention blocks of the decode step's
    launches (the library's diagnostic trace, 100 MHz clock), one launch at a
    time: the front launch's attention blocks and the sparse launch.  For
    each source kind, the median over blocks and the maximum of every phase,
    in microseconds after the first traced block of the launch started;
    medians over `reps` steps on the rotated layers.  Written as markdown to
    `path`."""
    import ctypes
    import torch
    from long_context_attention_20_amd import _lib
    words = 16 * 65536
    buf = torch.zeros(words, dtype=torch.int64, device="cuda:0")
    recs = {0: [], 1: []}
    try:
        for rep in range(reps):
            calls = run.calls(run.layers[rep % len(run.layers)])
            for j, f in enumerate(calls):
                traced = j in recs
                if traced:
                    buf.zero_()
                    torch.cuda.synchronize()
                    _lib.check(_lib.lib.lca_diag_trace(ctypes.c_void_p(buf.data_ptr()), words), "diag_trace")
                f()
                if traced:
                    torch.cuda.synchronize()
                    _lib.check(_lib.lib.lca_diag_trace(None, 0), "diag_trace")
                    rec = buf.view(-1, 16).cpu().numpy().view(np.uint64).astype(np.int64)
                    recs[j].append(rec[rec[:, 0] != 0])
            torch.cuda.synchronize()
    finally:
        _lib.lib.lca_diag_trace(None, 0)
    tick_us = 0.01
    out = []
    for j, title in ((0, run.names[0]), (1, run.names[1])):
        per_rep = [r for r in recs[j] if len(r)]
        if not per_rep:
            continue
        kinds = sorted(set(int(k) for r in per_rep for k in (r[:, 7] & 3)))
        lines = [f"### {title}", "",
                 "| source | blocks | " + " | ".join(f"{p} (median / max)" for p in TRACE_PHASES) + " |",
                 "|---|---|" + "---|" * len(TRACE_PHASES)]
        for kd in kinds:
            cells = []
            for ph in range(7):
                med, mx = [], []
                for r in per_rep:
                    t0 = r[:, 0].min()
                    v = r[(r[:, 7] & 3) == kd][:, ph]
                    v = v[v != 0]
                    if len(v):
                        med.append(np.median(v - t0) * tick_us)
                        mx.append(np.max(v - t0) * tick_us)
                cells.append(f"{np.median(med):.2f} / {np.median(mx):.2f}" if med else "-")
            nb = int(np.median([np.sum((r[:, 7] & 3) == kd) for r in per_rep]))
            lines.append(f"| {KIND_NAMES.get(kd, kd)} | {nb} | " + " | ".join(cells) + " |")
        sub = [(ph, nm) for ph, nm in SUB_PHASES]
        topk = [r[(r[:, 7] & 3) == 3] for r in per_rep]
        if any(len(t) for t in topk):
            cells = []
            for ph, nm in sub:
                med, mx = [], []
                for r, t in zip(per_rep, topk):
                    v = t[:, ph]
                    v = v[v != 0]
                    if len(v):
                        med.append(np.median(v - r[:, 0].min()) * tick_us)
                        mx.append(np.max(v - r[:, 0].min()) * tick_us)
                cells.append(f"{np.median(med):.2f} / {np.median(mx):.2f}" if med else "-")
            lines += ["", "top-k steps of the sparse blocks (median / max, us after the first block start):", "",
                      "| " + " | ".join(nm for _, nm in sub) + " |", "|" + "---|" * len(sub),
                      "| " + " | ".join(cells) + " |"]
        spans = [(r[:, 6].max() - r[:, 0].min()) * tick_us for r in per_rep]
        gave_up = sum(int(np.sum((r[:, 7] >> 2) & 1)) for r in per_rep)
        lines.append("")
        lines.append(f"first traced block start to last partial stored: median {np.median(spans):.2f} us over "
                     f"{len(per_rep)} steps; waits that gave up: {gave_up}")
        out.append("\n".join(lines))
    text = "\n\n".join(out) + "\n"
    with open(path, "w") as f:
        f.write(text)
    print(text, file=sys.stderr, flush=True)


def _host_info():
    """The host's CPU model and hardware thread count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        return 1


def _host_seq(raw, b, cfg):
    """Sequence b's raw streams on the host (float64): x, a, g, u, c and the
    option streams the workload has."""
    from oracle import pipeline as opipe
    off = raw["tok_off"].cpu().numpy()
    host = lambda t: t[int(off[b]):int(off[b + 1])].float().cpu().numpy().astype(np.float64)  # noqa: E731
    seq = {k: host(raw[k]) for k in ("x", "a", "g", "u", "c")}
    opt = {k: host(raw[k]) for k in opipe.OPTION_STREAMS if k in raw}
    return seq, opt


def _timed(fn, budget_s, cap):
    """Calls fn() until budget_s seconds or cap calls; (calls, seconds)."""
    n = 0
    t0 = time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= cap:
            return n, el


def _with_one_thread(fn):
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        return None
    with threadpool_limits(limits=1):
        return fn()


def cpu_baseline(cfg, state, budget_s):
    """The oracle (float64, numpy) on this host: one decode step per query of
    layer 0 -- append the completed entries, score, select, attend, merge --
    on caches it builds itself from the same raw inputs (build not timed);
    timed with the BLAS threads numpy starts with, then with one thread."""
    from oracle import compress as ocmp
    from oracle import numerics as onum
    from oracle import pipeline as opipe
    from oracle import quant as oquant
    threads = _blas_threads()
    raw = state.raw
    b = 0
    L = cfg.lens[b]
    t0 = time.perf_counter()
    seq, opt = _host_seq(raw, b, cfg)
    x, a, g, u, c = (seq[k] for k in ("x", "a", "g", "u", "c"))
    caches = opipe.build_seq_caches(x, a, g, u, c, cfg, opt)
    build_s = time.perf_counter() - t0
    tq = cfg.tq
    rows = []
    for t in range(tq):
        r = b * tq + t
        rows.append((raw["q"][r].float().cpu().numpy().astype(np.float64),
                     raw["p"][r].float().cpu().numpy().astype(np.float64),
                     raw["omega"][r].cpu().numpy().astype(np.float64), L - tq + t))
    sg = raw["sigma"].cpu().numpy().astype(np.float64)
    dual = (lambda k: opt[k]) if cfg.dual else (lambda k: None)  # noqa: E731

    def step():
        # append: the entries the step's tokens complete
        def new(m, w):
            return list(range(ocmp.n_entries(L - tq, m, w), ocmp.n_entries(L, m, w)))
        j = new(cfg.m, cfg.w)
        if j:
            caches.kv_csa[j] = opipe.kv_entries(x, a, cfg.m, cfg.w, cfg, j, dual("x_b"), dual("a_b"))
            pooled = ocmp.compress(u, c, cfg.m, cfg.w, False, cfg.eps, j, src2=dual("u_b"), z2=dual("c_b"))
            caches.ikey[j] = (oquant.dequantize_rows(*oquant.quantize_rows(pooled)) if cfg.ikey == "fp8" else
                              oquant.dequantize_mx_rows(*oquant.quantize_mx_rows(pooled)) if cfg.ikey == "mxfp4"
                              else onum.round_to(pooled, cfg.dtype))
            if cfg.sepv:
                caches.v_csa[j] = opipe.kv_entries(opt["v"], a, cfg.m, cfg.w, cfg, j, dual("v_b"), dual("a_b"))
        j = new(cfg.m2, cfg.w2)
        if j:
            caches.kv_hca[j] = opipe.kv_entries(x, g, cfg.m2, cfg.w2, cfg, j)
            if cfg.sepv:
                caches.v_hca[j] = opipe.kv_entries(opt["v"], g, cfg.m2, cfg.w2, cfg, j)
        for q, p, om, i in rows:
            opipe.query_step(caches, x, q, p, om, sg, i, cfg, v_seq=opt.get("v"))

    n, el = _timed(step, budget_s, 1000)
    one = _with_one_thread(lambda: _timed(step, budget_s / 3, 1000))
    model, hw = _host_info()
    where = f"1 query at position {L - 1}" if tq == 1 else f"{tq} queries at positions {L - tq}..{L - 1}"
    return {"value": n * tq / el, "unit": "q-tok/s/layer", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} decode steps of sequence 0 ({where}) of layer 0, float64 numpy oracle "
                      f"(append + indexer + top-k + sparse + HCA + window + sink + merge) on caches it built "
                      f"itself in {build_s:.1f} s (not timed); {el:.1f} s timed with {threads} BLAS threads",
            "seconds": round(el, 3),
            "value_1_thread": (one[0] * tq / one[1]) if one else None,
            "seconds_1_thread": round(one[1], 3) if one else None,
            "host_cpu": model, "host_threads": hw}


def cpu_baseline_prefill(cfg, raw, budget_s):
    """The oracle on this host for the prefill chunk: query rows of the chunk
    spread evenly over it (first and last included), each scored, selected
    and attended on caches the oracle builds from the whole context (build
    not timed)."""
    from oracle import pipeline as opipe
    threads = _blas_threads()
    b = 0
    L = cfg.lens[b]
    t0 = time.perf_counter()
    seq, opt = _host_seq(raw, b, cfg)
    caches = opipe.build_seq_caches(seq["x"], seq["a"], seq["g"], seq["u"], seq["c"], cfg, opt)
    build_s = time.perf_counter() - t0
    sg = raw["sigma"].cpu().numpy().astype(np.float64)
    order = np.unique(np.linspace(0, cfg.tq - 1, 257).astype(int))
    q = raw["q"].float().cpu().numpy()
    p = raw["p"].float().cpu().numpy()
    om = raw["omega"].cpu().numpy()
    state = {"k": 0}

    def row():
        t = int(order[state["k"] % len(order)])
        state["k"] += 1
        opipe.query_step(caches, seq["x"], q[t].astype(np.float64), p[t].astype(np.float64),
                         om[t].astype(np.float64), sg, L - cfg.tq + t, cfg, v_seq=opt.get("v"))

    n, el = _timed(row, budget_s, len(order))
    state["k"] = 0
    one = _with_one_thread(lambda: _timed(row, budget_s / 3, len(order)))
    model, hw = _host_info()
    return {"value": n / el, "unit": "q-tok/s/layer", "cores": threads, "kind": "oracle",
            "sample": f"{n} query rows of the {cfg.tq}-row chunk (evenly spaced, from the first), float64 numpy "
                      f"oracle (indexer + top-k + sparse + HCA + window + sink + merge) on caches of the whole "
                      f"{L}-token context it built itself in {build_s:.1f} s (not timed); {el:.1f} s timed with "
                      f"{threads} BLAS threads",
            "seconds": round(el, 3),
            "value_1_thread": (one[0] / one[1]) if one else None,
            "seconds_1_thread": round(one[1], 3) if one else None,
            "host_cpu": model, "host_threads": hw}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=24)
    ap.add_argument("--config", default="pro_1m_decode")
    ap.add_argument("--layers", type=int, default=0, help="layers to rotate over (0: enough to exceed 2x MALL)")
    ap.add_argument("--graph", type=int, default=1, help="1: headline from HIP graph replay")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle timing budget (0 disables)")
    ap.add_argument("--split-csa", type=int, default=0, help="entry splits of the sparse attention (0: default)")
    ap.add_argument("--split-hca", type=int, default=0, help="entry splits of the HCA attention (0: default)")
    ap.add_argument("--batch-invariant", type=int, default=0,
                    help="1: batch-invariant decode (fixed key ranges per split, HybridAttention(batch_invariant=True))")
    ap.add_argument("--half-partials", type=int, default=1,
                    help="1: the decode step's attention partials in fp16 (default), 0: fp32")
    ap.add_argument("--front", type=int, default=-1,
                    help="1: decode step in front form (HCA and window beside the scores), 0: HCA and window "
                         "beside the sparse blocks; -1: the layer's default for the workload")
    ap.add_argument("--trace-attn", default="", metavar="PATH",
                    help="also write the attention launch's per-block phase timeline to PATH")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB 10 times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "bench.py measures one GPU; --gpus must be 1 "
                                   "(the path has no multi-GPU sharding)"}))
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 10}))
        return
    import lca_inputs as li
    cfg = li.CONFIGS[args.config]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if cfg.tq > MTP_MAX_ROWS:
        run_prefill(cfg, args, dev)
        return
    sb = step_bytes(cfg)
    R = args.layers or max(1, -(-2 * MALL_BYTES // sb))
    t0 = time.perf_counter()
    run = Runner(cfg, R, dev, args.split_csa, args.split_hca, front=None if args.front < 0 else bool(args.front),
                 half_partials=bool(args.half_partials), batch_invariant=bool(args.batch_invariant))
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    print(f"[bench] {cfg.name}: {R} layers built in {setup_s:.1f} s; {sb / 1e6:.2f} MB/step; "
          f"splits csa={run.sc} hca={run.sh} window={run.sw}", file=sys.stderr, flush=True)

    # per-kernel durations: each single-kernel call captured R times (one per
    # rotated layer) in a HIP graph, replayed, timed with events on its stream
    s = torch.cuda.current_stream()
    for w in range(2 * R):
        run.step_calls(run.layers[w % R])
    torch.cuda.synchronize()
    tper = np.zeros(len(run.timed))
    reps = 8
    for i, tname in enumerate(run.timed):
        calls = [run.timed_call(L, tname) for L in run.layers]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in calls:
                f()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        tper[i] = e0.elapsed_time(e1) / (reps * R)
        del g
    tt = dict(zip(run.timed, tper))
    if args.trace_attn:
        trace_attention(run, args.trace_attn)
    def own_time(n):
        for key in run.timed:
            if key == n:
                return tt[key]
            if key.endswith("+" + n):
                return tt[key] - tt[key[:-len(n) - 1]]
        raise KeyError(n)
    per = np.array([own_time(n) for n in run.names])
    # the dominant kernel: the longest single launch
    dom = int(np.argmax([t / run.launches.get(n, 1) for n, t in zip(run.names, per)]))
    print("[bench] per-kernel ms (graph, rotated layers): " +
          ", ".join(f"{n}={t:.4f}" for n, t in zip(run.names, per)), file=sys.stderr, flush=True)

    K = args.steps
    # one sequence: the K timed steps are K consecutive decode steps ending at
    # L-1, each taking the next tq tokens (each appends what its tokens
    # complete: a CSA and an indexer entry every 4th token, an HCA entry every
    # 128th); several sequences: every step is the last position (all three
    # appends each step)
    tq = cfg.tq
    consecutive = cfg.B == 1 and cfg.lens[0] > tq * (K + args.warmup) + 2 * cfg.w2
    last = cfg.lens[0] - 1
    pos_t = [Position(last - tq * (K - 1 - it), dev, tq) for it in range(K)] if consecutive else [None] * K
    pos_w = [Position(last - tq * (K + args.warmup - 1 - w), dev, tq) for w in range(args.warmup)] if consecutive \
        else [None] * args.warmup
    ms_graph = ms_last = None
    if args.graph:
        # the warmup steps and the K timed steps each captured as one graph of
        # consecutive layer steps (as the layers of one forward pass run), so
        # that host-side launch cost is paid once per graph, not per step
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            for L in run.layers:
                run.step(L)
        torch.cuda.current_stream().wait_stream(s2)
        torch.cuda.synchronize()
        gw, gk, gl = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw):
            for w in range(args.warmup):
                run.step(run.layers[w % R], pos_w[w])
        with torch.cuda.graph(gk):
            for it in range(K):
                run.step(run.layers[it % R], pos_t[it])
        with torch.cuda.graph(gl):  # the last position: every append in every step
            for it in range(2 * R):
                run.step(run.layers[it % R])
        gw.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        gk.replay()
        e1.record()
        torch.cuda.synchronize()
        ms_graph = e0.elapsed_time(e1) / K
        gl.replay()
        torch.cuda.synchronize()
        e0.record()
        gl.replay()
        e1.record()
        torch.cuda.synchronize()
        ms_last = e0.elapsed_time(e1) / (2 * R)
        del gw, gk, gl

    # the same steps launched directly on one stream
    for w in range(args.warmup):
        run.step(run.layers[w % R], pos_w[w])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for it in range(K):
        run.step(run.layers[it % R], pos_t[it])
    e1.record()
    torch.cuda.synchronize()
    ms_stream = e0.elapsed_time(e1) / K
    k_ms = float(per[dom])

    ms = ms_graph if ms_graph is not None else ms_stream
    value = cfg.B * cfg.tq / (ms / 1e3)
    name = run.names[dom]
    kb, kf, kov = kernel_cost(cfg, name.split("(")[0], run.front)
    if kf / max(kb, 1) >= MFMA_BF16_PEAK / HBM_PEAK:
        roof = {"bound": "mfma", "achieved": kf / (k_ms / 1e3) / 1e12, "peak": MFMA_BF16_PEAK / 1e12,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": kb / (k_ms / 1e3) / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(cfg.name, name)
    roof["kernel"] = name
    roof["kernel_ms"] = k_ms
    roof["bytes_per_launch"] = kb
    roof["flops_per_launch"] = kf
    roof["overhead_bytes_per_launch"] = kov
    # every launch of the step against its share of the algorithmic bytes
    per_kernel = {}
    for n, t in zip(run.names, per):
        b_, f_, o_ = kernel_cost(cfg, n, run.front)
        per_kernel[n] = {"ms": float(t), "bytes": b_, "overhead_bytes": o_, "flops": f_,
                         "hbm_frac": b_ / (t / 1e3) / HBM_PEAK if t > 0 else None}

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(cfg, run.layers[0], args.cpu_seconds)

    res = {
        "metric": metric_name(cfg),
        "value": value,
        "unit": "q-tok/s/layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1), generated on the GPU)",
        "config": {"workload": cfg.name, "sequences": cfg.B, "context": list(cfg.lens) if cfg.B <= 8 else
                   f"{cfg.B} seqs, mean {int(np.mean(cfg.lens))}", "q_heads": cfg.H, "head_dim": cfg.D,
                   "indexer": f"{cfg.HI}x{cfg.dI}", "topk": cfg.k, "m": cfg.m, "m2": cfg.m2, "window": cfg.W,
                   "layers_rotated": R, "timing": "hip-graph replay" if ms_graph is not None else "stream",
                   "query_rows_per_step": tq, "indexer_keys": cfg.ikey,
                   "positions": (f"{K} consecutive decode steps over positions {last - tq * K + 1}..{last}, "
                                 f"{tq} per step, each appending the entries its tokens complete") if consecutive else
                   "last position of every sequence, every append in every step"},
        "hbm_frac_of_peak": sb / (ms / 1e3) / HBM_PEAK,
        "bytes_per_step": sb,
        "ms_per_step_stream": ms_stream,
        "ms_step_all_appends": ms_last,
        "kernel_ms": {n: float(t) for n, t in zip(run.names, per)},
        "kernels": per_kernel,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()
