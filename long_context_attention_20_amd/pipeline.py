"""One layer of hybrid compressed attention driven through liblca.

Holds the static shape of a layer (heads, head dim, indexer shape, top-k,
strides and windows), the caller's caches as device tensors with their host
and device offsets, and reusable workspaces.  It only sizes buffers and
sequences the C entry points; every step runs in the HIP kernels.

Decode step (one query row per sequence, or a few), three calls on one stream:
    decode_front  the CSA, indexer-key and HCA entries the new token
                  completes, the index scores, and the attention over the HCA
                  entries that existed before the step and over the window
                  (one launch: the attention blocks run beside the score blocks)
    hybrid_attn   exact top-k (every sparse block filters a share of the
                  scores, then selects its share of the ascending list) and
                  the sparse attention over it; the HCA entry the step
                  completes, when it completes one
    swa_merge     sink + merge of every partial
Prefill chunks (many rows per sequence) run kv_compress, csa_index_topk (the
scores and a streaming exact top-k in one launch, no score stored) and
hybrid_attn_merge.
"""
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import ops


def n_windows(L: int, m: int, w: int) -> int:
    """Complete windows of length w at stride m in L tokens (host-side sizing)."""
    return 0 if L < w else (L - w) // m + 1


@dataclass
class Caches:
    lens: List[int]          # tokens per sequence covered by the caches
    csa_off: torch.Tensor    # int64 [B+1]
    hca_off: torch.Tensor
    kv_csa: torch.Tensor     # [sum N_csa, D]
    ikey: torch.Tensor       # [sum N_csa, dI]
    kv_hca: torch.Tensor     # [sum N_hca, D]
    csa_off_h: np.ndarray
    hca_off_h: np.ndarray
    v_csa: Optional[torch.Tensor] = None   # value entries (separate values), rows as kv_csa
    v_hca: Optional[torch.Tensor] = None


def _offsets(counts) -> np.ndarray:
    o = np.zeros(len(counts) + 1, dtype=np.int64)
    o[1:] = np.cumsum(np.asarray(counts, dtype=np.int64))
    return o


class HybridAttention:
    def __init__(self, H: int, D: int, HI: int, dI: int, k: int, m: int = 4, w: int = 8, m2: int = 128,
                 w2: int = 128, W: int = 128, eps: float = 1e-6, scale: Optional[float] = None,
                 split_csa: Optional[int] = None, split_hca: Optional[int] = None, ikey: str = "bf16",
                 rope: int = 0, rope_base: float = 10000.0, dual: bool = False, sepv: bool = False,
                 batch_invariant: bool = False, max_context: int = 1 << 20, half_partials: bool = True):
        self.H, self.D, self.HI, self.dI, self.k = H, D, HI, dI, k
        # half_partials: decode_step keeps the attention partials it merges
        # as fp16 (bf16 inputs, H a multiple of 16); every partial is a convex
        # combination of RMS-normalised value rows, far inside fp16's range
        self.half_partials = bool(half_partials)
        # partial rotary embedding on the last `rope` dims of each head (0:
        # none): compressed entries are stored turned by the position of
        # their window's last token, queries and window tokens turn by their
        # own positions, and every attention output is turned back by the
        # query position; indexer keys and queries are not turned
        if rope < 0 or rope % 2 or rope > D:
            raise ValueError(f"rope: an even number of dims <= D, not {rope}")
        self.rope, self.rope_base = int(rope), float(rope_base)
        # dual: the CSA windows (KV, values and indexer keys) pool their last
        # m tokens from second-half streams (raw inputs x_b, a_b, u_b, c_b,
        # and v_b with separate values); needs w = 2m.  sepv: values from
        # the raw stream v, pooled with the keys' logits (value caches
        # v_csa, v_hca), the window's values the raw v tokens
        if dual and w != 2 * m:
            raise ValueError("the dual-stream compressor needs w = 2m")
        self.dual, self.sepv = bool(dual), bool(sepv)
        # batch_invariant: a decode step gives every sequence the same output
        # bits alone and inside any batch (invariant_splits); max_context
        # bounds the contexts the layer serves (it fixes the split counts)
        self.batch_invariant, self.max_context = bool(batch_invariant), int(max_context)
        # indexer-key cache: rows of the inputs' type ("bf16"), fp8 rows (d_I
        # E4M3 bytes, fp32 scale, 4 zero bytes) or MXFP4 rows (d_I/2 bytes of
        # E2M1 pairs, one E8M0 scale per 32 channels, zero pad to d_I/2 + 8)
        if ikey not in ("bf16", "fp8", "mxfp4"):
            raise ValueError(f"ikey: bf16, fp8 or mxfp4, not {ikey}")
        self.ikey = ikey
        self.ikey_code = {"bf16": 0, "fp8": 1, "mxfp4": 2}[ikey]
        self.m, self.w, self.m2, self.w2, self.W, self.eps = m, w, m2, w2, W, eps
        self.scale = float(scale) if scale is not None else 1.0 / float(np.sqrt(D))
        self.split_csa, self.split_hca = split_csa, split_hca
        self._ws: Dict[str, torch.Tensor] = {}

    # -------------------------------------------------------------- buffers
    def _workspace(self, name: str, nbytes: int, device, zero: bool) -> torch.Tensor:
        t = self._ws.get(name)
        if t is None or t.numel() < nbytes or t.device != torch.device(device):
            t = (torch.zeros if zero else torch.empty)(max(nbytes, 256), dtype=torch.uint8, device=device)
            self._ws[name] = t
        return t

    def alloc_caches(self, lens: Sequence[int], device, dtype) -> Caches:
        lens = [int(v) for v in lens]
        co = _offsets([n_windows(L, self.m, self.w) for L in lens])
        ho = _offsets([n_windows(L, self.m2, self.w2) for L in lens])
        return Caches(
            lens=lens,
            csa_off=torch.from_numpy(co).to(device), hca_off=torch.from_numpy(ho).to(device),
            # at least one row each, so that empty caches still have an address
            kv_csa=torch.empty((max(1, int(co[-1])), self.D), dtype=dtype, device=device),
            ikey=(torch.empty((max(1, int(co[-1])), self.dI + 8 if self.ikey == "fp8" else self.dI // 2 + 8),
                              dtype=torch.uint8, device=device) if self.ikey_code
                  else torch.empty((max(1, int(co[-1])), self.dI), dtype=dtype, device=device)),
            kv_hca=torch.empty((max(1, int(ho[-1])), self.D), dtype=dtype, device=device),
            csa_off_h=co, hca_off_h=ho,
            v_csa=torch.empty((max(1, int(co[-1])), self.D), dtype=dtype, device=device) if self.sepv else None,
            v_hca=torch.empty((max(1, int(ho[-1])), self.D), dtype=dtype, device=device) if self.sepv else None)

    def _values(self, srcs, caches: Caches, v: Optional[torch.Tensor]):
        """Attention sources with their value rows (separate values): the
        value caches beside the CSA and HCA entries, the raw value tokens
        beside the window's."""
        if self.sepv:
            if v is None:
                raise ValueError("separate values: the raw value tokens v are required")
            for d in srcs:
                d["v"] = {"topk": caches.v_csa, "gather": caches.v_csa, "dense": caches.v_hca, "window": v}[d["kind"]]
        return srcs

    def _turn(self, d: dict) -> dict:
        """A compression stream or attention source with the layer's rotary
        embedding."""
        if self.rope:
            d.update(rope=self.rope, rope_base=self.rope_base)
        return d

    # -------------------------------------------------------------- compression
    def compress_streams(self, caches: Caches, raw: dict, done_h: Sequence[int], which=("csa", "idx", "hca"),
                         lens_h: Optional[Sequence[int]] = None):
        """Descriptors of the entries completed after done_h[b] tokens (up to
        lens_h[b] tokens, default the caches' lengths; the sizes only bound
        the launch, the kernels read the lengths from tok_off)."""
        lens = caches.lens if lens_h is None else lens_h
        new_csa = max(n_windows(L, self.m, self.w) - n_windows(d, self.m, self.w) for L, d in zip(lens, done_h))
        new_hca = max(n_windows(L, self.m2, self.w2) - n_windows(d, self.m2, self.w2) for L, d in zip(lens, done_h))
        sec = (lambda s, z: dict(src2=raw[s], logits2=raw[z])) if self.dual else (lambda s, z: {})  # noqa: E731
        streams = []
        if new_csa > 0 and "csa" in which:
            streams.append(self._turn(dict(src=raw["x"], logits=raw["a"], out=caches.kv_csa, ent_off=caches.csa_off,
                                           m=self.m, w=self.w, rmsnorm=1, max_entries=new_csa, **sec("x_b", "a_b"))))
            if self.sepv:
                streams.append(self._turn(dict(src=raw["v"], logits=raw["a"], out=caches.v_csa,
                                               ent_off=caches.csa_off, m=self.m, w=self.w, rmsnorm=1,
                                               max_entries=new_csa, **sec("v_b", "a_b"))))
        if new_csa > 0 and "idx" in which:
            streams.append(dict(src=raw["u"], logits=raw["c"], out=caches.ikey, ent_off=caches.csa_off,
                                m=self.m, w=self.w, rmsnorm=0, max_entries=new_csa, key=self.ikey_code,
                                **sec("u_b", "c_b")))
        if new_hca > 0 and "hca" in which:
            streams.append(self._turn(dict(src=raw["x"], logits=raw["g"], out=caches.kv_hca, ent_off=caches.hca_off,
                                           m=self.m2, w=self.w2, rmsnorm=1, max_entries=new_hca)))
            if self.sepv:
                streams.append(self._turn(dict(src=raw["v"], logits=raw["g"], out=caches.v_hca,
                                               ent_off=caches.hca_off, m=self.m2, w=self.w2, rmsnorm=1,
                                               max_entries=new_hca)))
        return streams

    @staticmethod
    def _launch_groups(streams):
        """The streams as kv_compress calls: one vector width and at most four
        streams per call."""
        groups: Dict[int, list] = {}
        for s in streams:
            lanes = s["src"].shape[-1] // (8 if s["src"].dtype == torch.bfloat16 else 4)
            groups.setdefault(1 if lanes <= 64 else lanes // 64, []).append(s)
        return [g[i:i + 4] for g in groups.values() for i in range(0, len(g), 4)]

    def compress(self, caches: Caches, raw: dict, tok_off: torch.Tensor,
                 done_len: Optional[torch.Tensor] = None, done_len_h: Optional[Sequence[int]] = None,
                 which=("csa", "idx", "hca")):
        """Write the entries of every sequence completed after done_len tokens
        (all of them when done_len is None)."""
        done = [0] * len(caches.lens) if done_len_h is None else [int(v) for v in done_len_h]
        streams = self.compress_streams(caches, raw, done, which)
        for g in self._launch_groups(streams):
            ops.kv_compress(g, tok_off, done_len, self.eps)

    def _append(self, caches: Caches, raw: dict, tok_off, done_len, done_h, which=("csa", "idx", "hca"),
                lens_h=None):
        """Launch the compression of the entries completed after done_h tokens
        (one launch when the streams share a vector width)."""
        streams = self.compress_streams(caches, raw, done_h, which, lens_h)
        for g in self._launch_groups(streams):
            ops.kv_compress(g, tok_off, done_len, self.eps)

    # -------------------------------------------------------------- indexer, top-k, attention
    def index_workspace(self, rows: int, max_entries: int, device) -> torch.Tensor:
        nbytes = ops.csa_index_topk_workspace(rows, max(1, max_entries), self.k)
        return self._workspace(f"idx{rows}_{max_entries}", nbytes, device, zero=True)

    def default_splits(self, rows: int, n_keys: int) -> int:
        """Splits of one source launched on its own: about one block per
        compute unit, at least two tiles for each of a block's two streams."""
        hg = (self.H + 31) // 32
        tiles = max(1, (n_keys + 31) // 32)
        want = max(1, -(-256 // (rows * hg)))
        return int(max(1, min(want, tiles // 4 if tiles >= 4 else 1, 256)))

    # batch-invariant decode: 32-key tiles per split of the sparse and the
    # HCA source
    INV_TILES = (2, 4)

    def invariant_splits(self):
        """Splits of a batch-invariant decode step: every split of a source
        takes a fixed range of a row's keys (tiles_per_split: 64 selected
        entries, 128 HCA entries; the window whole) and the split counts
        follow from k and max_context alone, so a row's partials, the merge's
        slot layout and its summation order do not depend on the other rows
        of the call; more than 16 slots in all, so that the merge is the same
        kernel for any number of rows."""
        sc = -(-self.k // (32 * self.INV_TILES[0]))
        sh = max(1, -(-n_windows(self.max_context, self.m2, self.w2) // (32 * self.INV_TILES[1])))
        sw = 1
        sh = max(sh, 17 - sc - sw)
        return sc, sh, sw

    # the row's scores a sparse block filters in one pass when it selects:
    # chunks of 512 threads x 8 scores, two chunks loaded at the block's start
    FILTER_PASS_SCORES = 2 * 512 * 8

    def fused_splits(self, rows: int, n_csa: int, n_hca: int, n_win: int, select: bool = False,
                     n_scores: int = 0):
        """Splits of the three sources of one fused launch: the blocks of all
        sources take about the same number of 32-key tiles (an even number,
        one per team and round), the fewest that let one wave of blocks (one
        per compute unit) cover the launch when the rows allow it.  With
        select, the sparse blocks also run the top-k selection (about as long
        as four tiles of attention) and take four tiles fewer, and there are
        enough of them that each filters its share of the row's n_scores
        scores in one pass."""
        hg = (self.H + 31) // 32
        if rows * hg >= 256:
            # the rows alone give the device a wave of blocks (and the dense
            # branch then runs row-tiled): one partial per source
            return (1, 1, 1)
        tiles = [max(1, (n + 31) // 32) for n in (n_csa, n_hca, n_win)]
        if self.rope:
            # a window tile is RMS-normalised and turned by the rotary
            # embedding as it is staged: measured about four times an HCA
            # tile, so the window takes more splits
            tiles[2] *= 4
        budget = max(3, 256 // max(1, rows * hg))
        sc_min = -(-n_scores // (self.FILTER_PASS_SCORES * hg)) if select else 1
        for floor in (sc_min, 1):  # a floor that does not fit the budget is dropped
            for per in range(2, 34, 2):
                pc = max(2, per - 4) if select else per
                sc = max(-(-tiles[0] // pc), floor)
                units = sc + -(-tiles[1] // per) + -(-tiles[2] // per)
                if units <= budget:
                    break
            if units <= budget:
                break
        return (int(min(256, max(1, sc))), int(min(256, max(1, -(-tiles[1] // per)))),
                int(min(256, max(1, -(-tiles[2] // per)))))

    def step(self, caches: Caches, x: torch.Tensor, tok_off: torch.Tensor, q: torch.Tensor, p: torch.Tensor,
             omega: torch.Tensor, sigma: Optional[torch.Tensor], q_pos: torch.Tensor, q_pos_h: np.ndarray,
             mode: str = "A", keep: bool = False, v: Optional[torch.Tensor] = None):
        """Attention output for every query row (after the caches hold every
        entry the query positions can see).  mode "A": one softmax over the
        selected CSA entries, the visible HCA entries, the window and the sink;
        "B": returns (csa-layer output, hca-layer output).  v: the raw value
        tokens (separate values)."""
        if self.sepv and v is None:
            raise ValueError("separate values: pass the raw value tokens v")
        rows = q.shape[0]
        dev = q.device
        qmax = int(np.max(q_pos_h)) + 1
        max_csa = max(1, n_windows(qmax, self.m, self.w))
        max_hca = n_windows(qmax, self.m2, self.w2)
        ws = self.index_workspace(rows, max_csa, dev)
        idx = ops.csa_index_topk(p, omega, caches.ikey, caches.csa_off, q_pos, self.k, self.m, self.w, max_csa, ws)
        wsm = self._workspace(f"swa{rows}", ops.swa_merge_workspace(rows, self.H, self.D), dev, zero=False)
        if mode == "A":
            # the three branches in one launch, merged with the sink
            sc, sh, sw = self.fused_splits(rows, min(self.k, max_csa), max_hca, self.W)
            sc, sh = self.split_csa or sc, self.split_hca or sh
            # the dense source is always launched (an empty one writes o = 0,
            # lse = -inf), so that the partials are there for every row
            bufs = dict(sc=sc, sh=sh, sw=sw, max_hca=1, csa=(None, None), hca=(None, None), swa=(None, None))
            srcs = self.attn_sources(caches, x, tok_off, idx, bufs, v)
            # attention and merge in one call (one launch when every source
            # has one split); with keep, the partials are computed as well
            out = ops.hybrid_attn_merge(q, q_pos, srcs, sigma, self.scale, self.eps)
            csa = hca = None
            if keep:
                parts = ops.hybrid_attn(q, q_pos, srcs, self.scale, self.eps)
                csa, hca = parts[0], parts[1]
        elif self.rope or self.sepv:
            # the per-branch calls take no rotary embedding and no separate
            # values: each layer is one merged call over its compressed
            # entries and the window
            sc = self.split_csa or self.default_splits(rows, self.k)
            sh = self.split_hca or self.default_splits(rows, max_hca)
            vals = lambda t: dict(v=t) if self.sepv else {}  # noqa: E731
            win = ([self._turn(dict(kind="window", kv=x, off=tok_off, W=self.W, n_split=1, **vals(v)))]
                   if self.W > 0 else [])
            csa_src = self._turn(dict(kind="gather", kv=caches.kv_csa, off=caches.csa_off, idx=idx, n_split=sc,
                                      **vals(caches.v_csa)))
            hca_src = self._turn(dict(kind="dense", kv=caches.kv_hca, off=caches.hca_off, m2=self.m2, w2=self.w2,
                                      n_split=sh, **vals(caches.v_hca)))
            o1 = ops.hybrid_attn_merge(q, q_pos, [csa_src] + win, sigma, self.scale, self.eps)
            o2 = ops.hybrid_attn_merge(q, q_pos, [hca_src] + win, sigma, self.scale, self.eps)
            out = (o1, o2)
            csa = hca = None
            if keep:
                csa = ops.hybrid_attn(q, q_pos, [csa_src], self.scale, self.eps)[0]
                hca = ops.hybrid_attn(q, q_pos, [hca_src], self.scale, self.eps)[0]
        else:
            sc = self.split_csa or self.default_splits(rows, self.k)
            sh = self.split_hca or self.default_splits(rows, max_hca)
            csa = ops.csa_sparse_attn(q, caches.kv_csa, caches.csa_off, idx, self.scale, self.eps, sc)
            hca = ops.hca_attn(q, caches.kv_hca, caches.hca_off, q_pos, self.m2, self.w2, max_hca, self.scale,
                               self.eps, sh)
            o1 = ops.swa_merge(q, x, tok_off, q_pos, sigma, [csa], self.W, self.scale, self.eps, wsm)
            o2 = ops.swa_merge(q, x, tok_off, q_pos, sigma, [hca], self.W, self.scale, self.eps, wsm)
            out = (o1, o2)
        if keep:
            return out, dict(idx=idx, csa=csa, hca=hca)
        return out

    def front_splits(self, rows: int, n_csa: int, n_hca: int, n_scores: int):
        """Splits of the decode step in front / sparse form: the HCA source
        runs beside the index scores (its blocks hold about half of the
        compute units there, the score blocks the rest); the sparse launch
        holds the sparse source alone, two 32-key tiles per block and enough
        blocks that each filters its share of the row's n_scores scores in
        one pass."""
        hg = (self.H + 31) // 32
        per_row = max(1, rows * hg)
        t_hca = max(1, (n_hca + 31) // 32)
        sh = max(1, min(t_hca // 4 if t_hca >= 4 else 1, 128 // per_row if per_row < 128 else 1, 256))
        t_csa = max(1, (n_csa + 31) // 32)
        sc = max(1, -(-t_csa // 2))
        sc = max(sc, -(-n_scores // (self.FILTER_PASS_SCORES * hg)))
        sc = max(1, min(sc, t_csa, 256 // per_row if per_row < 256 else 1))
        return int(sc), int(sh), 1

    # -------------------------------------------------------------- whole step
    def front_default(self, rows: int) -> bool:
        """Whether a decode step takes the front form by default: never on
        the measured workloads (Pro 1M, Pro varlen, Flash decode), where the
        HCA blocks beside the sparse blocks hide under the selection chain,
        while beside the score blocks they queue behind the key stream and
        lengthen the score launch by more than they take off the other."""
        return False

    def decode_buffers(self, rows: int, max_csa: int, max_hca: int, device, dtype, front: Optional[bool] = None):
        """Preallocated outputs of decode_step (so that the step can be
        captured in a HIP graph and replayed).  front: the front / sparse
        form of the step (decode_step then runs front_calls); None: the
        default for `rows` (front_default)."""
        if front is None:
            front = self.front_default(rows)
        f32 = torch.float32
        if self.batch_invariant:
            front = False
            sc, sh, sw = self.invariant_splits()
        elif front:
            sc, sh, sw = self.front_splits(rows, min(self.k, max(1, max_csa)), max_hca, max_csa)
        else:
            sc, sh, sw = self.fused_splits(rows, min(self.k, max(1, max_csa)), max_hca, self.W, select=True,
                                           n_scores=max_csa)
        if not self.batch_invariant:
            sc = self.split_csa or sc
            sh = self.split_hca or sh
        # fp16 partials (o_half) where the decode kernel writes them
        odt = torch.float16 if (self.half_partials and dtype == torch.bfloat16 and self.H % 16 == 0) else f32
        part = lambda n: (torch.empty((n, rows, self.H, self.D), dtype=odt, device=device),  # noqa: E731
                          torch.empty((n, rows, self.H), dtype=f32, device=device))
        return dict(
            sc=sc, sh=sh, sw=sw, max_csa=max(1, max_csa), max_hca=max_hca, front=front,
            ws_idx=self.index_workspace(rows, max(1, max_csa), device),
            idx=torch.empty((rows, self.k), dtype=torch.int32, device=device),
            csa=part(sc), hca=part(sh), swa=part(sw), hca_new=part(1),
            out=torch.empty((rows, self.H, self.D), dtype=dtype, device=device))

    def attn_sources(self, caches: Caches, x: torch.Tensor, tok_off: torch.Tensor, idx: Optional[torch.Tensor],
                     bufs: dict, v: Optional[torch.Tensor] = None):
        """The three key sources of the fused attention launch.  idx None: the
        sparse source selects its own entries from the index workspace
        bufs["ws_idx"] (a TOPK source; the selection lands in bufs["idx"]).
        v: the raw value tokens (separate values)."""
        if idx is None:
            src = [dict(kind="topk", kv=caches.kv_csa, off=caches.csa_off, k=self.k, m2=self.m, w2=self.w,
                        max_entries=bufs["max_csa"], ws=bufs["ws_idx"], idx_out=bufs["idx"], n_split=bufs["sc"],
                        o_part=bufs["csa"][0], lse=bufs["csa"][1])]
        else:
            src = [dict(kind="gather", kv=caches.kv_csa, off=caches.csa_off, idx=idx, n_split=bufs["sc"],
                        o_part=bufs["csa"][0], lse=bufs["csa"][1])]
        if bufs["max_hca"] > 0 or self.batch_invariant:  # (a fixed slot layout: always present)
            src.append(dict(kind="dense", kv=caches.kv_hca, off=caches.hca_off, m2=self.m2, w2=self.w2,
                            n_split=bufs["sh"], o_part=bufs["hca"][0], lse=bufs["hca"][1]))
        if self.W > 0:
            src.append(dict(kind="window", kv=x, off=tok_off, W=self.W, n_split=bufs["sw"], o_part=bufs["swa"][0],
                            lse=bufs["swa"][1]))
        if self.batch_invariant:
            tps = {"topk": self.INV_TILES[0], "gather": self.INV_TILES[0], "dense": self.INV_TILES[1],
                   "window": -(-self.W // 32)}
            for d in src:
                d["tiles_per_split"] = tps[d["kind"]]
        return [self._turn(d) for d in self._values(src, caches, v)]

    def front_calls(self, caches: Caches, raw: dict, tok_off: torch.Tensor, q, p, omega, sigma, q_pos, bufs: dict,
                    done_len: torch.Tensor, done_h: Sequence[int], lens_h: Optional[Sequence[int]] = None):
        """The decode step as three launches, returned as three callables (so
        that each can be timed on its own): decode_front (the appends of the
        entries the new tokens complete, the index scores, and the attention
        over the HCA entries that existed before the step and over the
        window), hybrid_attn (the exact top-k inside the sparse blocks, and
        the HCA entries the step completes, if any), swa_merge (every partial
        and the sink into bufs["out"])."""
        lens = caches.lens if lens_h is None else lens_h
        streams = self.compress_streams(caches, raw, done_h, lens_h=lens_h)
        idx_st = [st for st in streams if st["out"] is caches.ikey]
        kv_st = [st for st in streams if st["out"] is not caches.ikey]
        if not idx_st:  # no new indexer key: the stream appends nothing
            idx_st = [dict(src=raw["u"], logits=raw["c"], out=caches.ikey, ent_off=caches.csa_off, m=self.m,
                           w=self.w, rmsnorm=0, max_entries=0, key=self.ikey_code)]
        front, parts = [], [bufs["csa"]]
        if bufs["max_hca"] > 0:
            front.append(dict(kind="dense", kv=caches.kv_hca, off=caches.hca_off, m2=self.m2, w2=self.w2,
                              part=1, done_len=done_len, n_split=bufs["sh"], o_part=bufs["hca"][0],
                              lse=bufs["hca"][1]))
            parts.append(bufs["hca"])
        if self.W > 0:
            front.append(dict(kind="window", kv=raw["x"], off=tok_off, W=self.W, n_split=bufs["sw"],
                              o_part=bufs["swa"][0], lse=bufs["swa"][1]))
            parts.append(bufs["swa"])
        back = [dict(kind="topk", kv=caches.kv_csa, off=caches.csa_off, k=self.k, m2=self.m, w2=self.w,
                     max_entries=bufs["max_csa"], ws=bufs["ws_idx"], idx_out=bufs["idx"], n_split=bufs["sc"],
                     o_part=bufs["csa"][0], lse=bufs["csa"][1])]
        if bufs["max_hca"] > 0 and any(n_windows(L, self.m2, self.w2) > n_windows(d, self.m2, self.w2)
                                       for L, d in zip(lens, done_h)):
            back.append(dict(kind="dense", kv=caches.kv_hca, off=caches.hca_off, m2=self.m2, w2=self.w2, part=2,
                             done_len=done_len, n_split=1, o_part=bufs["hca_new"][0], lse=bufs["hca_new"][1]))
            parts.append(bufs["hca_new"])
        front = [self._turn(d) for d in self._values(front, caches, raw.get("v"))]
        back = [self._turn(d) for d in self._values(back, caches, raw.get("v"))]
        if not front:  # nothing to attend beside the scores
            f0 = lambda: ops.csa_index_score_append(p, omega, caches.ikey, caches.csa_off, q_pos, self.k, self.m,  # noqa: E731
                                                    self.w, bufs["max_csa"], bufs["ws_idx"], idx_st[0], kv_st,
                                                    tok_off, done_len, self.eps)
        else:
            f0 = lambda: ops.decode_front(p, omega, caches.ikey, caches.csa_off, q_pos, self.k, self.m, self.w,  # noqa: E731
                                          bufs["max_csa"], bufs["ws_idx"], idx_st[0], kv_st, tok_off, done_len, q,
                                          front, self.scale, self.eps)
        return [f0,
                lambda: ops.hybrid_attn(q, q_pos, back, self.scale, self.eps),
                lambda: ops.swa_merge(q, None, None, None, sigma, parts, 0, self.scale, self.eps, None,
                                      out=bufs["out"])]

    def decode_step(self, caches: Caches, raw: dict, tok_off: torch.Tensor, q, p, omega, sigma, q_pos,
                    bufs: dict, done_len: Optional[torch.Tensor] = None, done_h: Optional[Sequence[int]] = None,
                    side: Optional["torch.cuda.Stream"] = None, lens_h: Optional[Sequence[int]] = None,
                    fuse_topk: bool = True):
        """One decode (or prefill-chunk) step of mode A: append the entries the
        new tokens complete (when done_len is given), score and select the CSA
        entries, attend to the selected CSA entries, the visible HCA entries
        and the window in one launch, and merge the partials with the sink.
        With one query row per sequence the appends ride in the scoring
        launch.  With a side stream the HCA append runs there instead, beside
        the indexer (the join costs a cross-queue wait in a graph).  lens_h:
        host copy of the sequence lengths tok_off describes, when they are
        shorter than the caches'.  fuse_topk: the top-k selection runs
        inside the attention call (a TOPK source) rather than as
        csa_topk_select.  Buffers from decode_buffers(front=True) with
        done_len, one query row or a few per sequence, no side stream and
        the fused top-k: the three-launch front form (front_calls)."""
        rows_per_seq = q.shape[0] // len(caches.lens)
        if (bufs.get("front") and done_len is not None and side is None and fuse_topk and
                (rows_per_seq == 1 or (rows_per_seq <= 4 and rows_per_seq * self.HI <= 16))):
            for f in self.front_calls(caches, raw, tok_off, q, p, omega, sigma, q_pos, bufs, done_len, done_h,
                                      lens_h):
                f()
            return bufs["out"]
        main = torch.cuda.current_stream()
        join = None
        scored = False
        if done_len is not None:
            if side is not None:
                fork = torch.cuda.Event()
                fork.record(main)
                side.wait_event(fork)
                with torch.cuda.stream(side):
                    self._append(caches, raw, tok_off, done_len, done_h, ("hca",), lens_h)
                    join = torch.cuda.Event()
                    join.record(side)
                self._append(caches, raw, tok_off, done_len, done_h, ("csa", "idx"), lens_h)
            else:
                streams = self.compress_streams(caches, raw, done_h, lens_h=lens_h)
                idx_st = [st for st in streams if st["out"] is caches.ikey]
                kv_st = [st for st in streams if st["out"] is not caches.ikey]
                rows_per_seq = q.shape[0] // len(caches.lens)
                if idx_st and (rows_per_seq == 1 or (rows_per_seq <= 4 and rows_per_seq * self.HI <= 16)):
                    ops.csa_index_score_append(p, omega, caches.ikey, caches.csa_off, q_pos, self.k, self.m, self.w,
                                               bufs["max_csa"], bufs["ws_idx"], idx_st[0], kv_st, tok_off, done_len,
                                               self.eps)
                    scored = True
                else:
                    self._append(caches, raw, tok_off, done_len, done_h, lens_h=lens_h)
        if not scored:
            ops.csa_index_score(p, omega, caches.ikey, caches.csa_off, q_pos, self.k, self.m, self.w,
                                bufs["max_csa"], bufs["ws_idx"])
        if not fuse_topk:
            ops.csa_topk_select(caches.csa_off, q_pos, self.k, self.m, self.w, bufs["max_csa"], bufs["ws_idx"],
                                idx=bufs["idx"])
        if join is not None:
            main.wait_event(join)
        srcs = self.attn_sources(caches, raw["x"], tok_off, None if fuse_topk else bufs["idx"], bufs, raw.get("v"))
        parts = ops.hybrid_attn(q, q_pos, srcs, self.scale, self.eps)
        ops.swa_merge(q, None, None, None, sigma, parts, 0, self.scale, self.eps, None, out=bufs["out"])
        return bufs["out"]
