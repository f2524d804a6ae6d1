"""Torch-tensor front end of liblca: argument marshalling only.

Every function here takes device tensors, checks their dtype/device/layout,
and calls the C entry point of the same name on the current torch stream.
All arithmetic runs in the HIP kernels of liblca.so.
"""
from typing import Optional, Sequence

import ctypes
import torch

from ._lib import (LCA_BF16, LCA_BF16_FP8KEY, LCA_BF16_MXFP4KEY, LCA_F32, LCA_SRC_DENSE, LCA_SRC_GATHER, LCA_SRC_TOPK, LCA_SRC_WINDOW, AttnSource, CompressStream,
                   Partial, check, lib)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LCA_BF16
    if t.dtype == torch.float32:
        return LCA_F32
    raise TypeError(f"unsupported element type {t.dtype} (bfloat16 or float32)")


def _index_dtype(p: torch.Tensor, ikey: torch.Tensor) -> int:
    """Element type code of an index-score call: the query's type, or for a
    uint8 key cache LCA_BF16_FP8KEY (rows of d_I + 8 bytes) or
    LCA_BF16_MXFP4KEY (rows of d_I/2 + 8 bytes)."""
    if ikey.dtype == torch.uint8:
        dI = p.shape[-1]
        if p.dtype != torch.bfloat16 or ikey.dim() != 2 or ikey.shape[1] not in (dI + 8, dI // 2 + 8):
            raise TypeError("key rows: bf16 queries and a uint8 cache of d_I + 8 (fp8) or d_I/2 + 8 (MXFP4) bytes per row")
        return LCA_BF16_FP8KEY if ikey.shape[1] == dI + 8 else LCA_BF16_MXFP4KEY
    return _dtype_code(p)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _addr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("liblca takes device tensors")
        if not t.is_contiguous():
            raise ValueError("liblca takes contiguous tensors")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _i64(t: torch.Tensor, what: str):
    if t.dtype != torch.int64:
        raise TypeError(f"{what} must be int64")


def _i32(t: torch.Tensor, what: str):
    if t.dtype != torch.int32:
        raise TypeError(f"{what} must be int32")


# ---------------------------------------------------------------- compression

def _stream_array(streams: Sequence[dict]):
    """ctypes array of lca_compress_stream and the common element type."""
    arr = (CompressStream * max(1, len(streams)))()
    dt = None
    for i, s in enumerate(streams):
        src, lg, out, eo = s["src"], s["logits"], s["out"], s["ent_off"]
        _dev(src, lg, out, eo)
        _i64(eo, "ent_off")
        d = _dtype_code(src)
        if dt is None:
            dt = d
        key = int(s.get("key", 0))
        C = src.shape[-1]
        if key:
            # key rows: fp8 (C E4M3 bytes, fp32 scale, 4 zero bytes) or MXFP4
            # (C/2 bytes of E2M1 pairs, one E8M0 scale per 32 channels, pad)
            rb = C + 8 if key == 1 else C // 2 + 8
            if out.dtype != torch.uint8 or out.dim() != 2 or out.shape[1] != rb:
                raise TypeError(f"key rows: a uint8 output of {rb} bytes per row")
        elif _dtype_code(out) != d:
            raise TypeError("one element type per call")
        if d != dt or _dtype_code(lg) != d:
            raise TypeError("one element type per call")
        pc = 1 if lg.dim() == 2 else 0
        src2, lg2 = s.get("src2"), s.get("logits2")
        if (src2 is None) != (lg2 is None):
            raise ValueError("src2 and logits2 come together")
        if src2 is not None:
            _dev(src2, lg2)
            if src2.shape != src.shape or lg2.shape != lg.shape or _dtype_code(src2) != d or _dtype_code(lg2) != d:
                raise TypeError("second-half streams shaped and typed as the first")
        arr[i] = CompressStream(src.data_ptr(), lg.data_ptr(), out.data_ptr(), eo.data_ptr(), C, int(s["m"]),
                                int(s["w"]), pc, int(s["rmsnorm"]), int(s["max_entries"]), key,
                                int(s.get("rope", 0)), float(s.get("rope_base", 10000.0)), _addr(src2), _addr(lg2))
    return arr, dt


def kv_compress(streams: Sequence[dict], tok_off: torch.Tensor, done_len: Optional[torch.Tensor] = None,
                eps: float = 1e-6):
    """streams: dicts with src, logits, out, ent_off (tensors) and m, w,
    rmsnorm, max_entries (ints); per_channel is taken from the logits' rank."""
    if not 1 <= len(streams) <= 4:
        raise ValueError("1..4 streams per call")
    _i64(tok_off, "tok_off")
    B = tok_off.numel() - 1
    arr, dt = _stream_array(streams)
    _dev(tok_off, done_len)
    if done_len is not None:
        _i64(done_len, "done_len")
    check(lib.lca_kv_compress(arr, len(streams), _ptr(tok_off), _ptr(done_len), B, float(eps), dt, _stream()),
          "kv_compress")


# ---------------------------------------------------------------- indexer + top-k

def csa_index_topk_workspace(n_rows: int, max_entries: int, k: int) -> int:
    return int(lib.lca_csa_index_topk_workspace(n_rows, max_entries, k))


def csa_index_topk(p, omega, ikey, csa_off, q_pos, k: int, m: int, w: int, max_entries: int, ws: torch.Tensor,
                   idx: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None):
    """p [B*Tq, H_I, d_I], omega [B*Tq, H_I] fp32, ikey [N, d_I], csa_off
    int64 [B+1], q_pos int32 [B, Tq].  Returns idx int32 [B*Tq, k]."""
    _dev(p, omega, ikey, csa_off, q_pos, ws, idx, scores)
    _i64(csa_off, "csa_off")
    _i32(q_pos, "q_pos")
    B = csa_off.numel() - 1
    rows = q_pos.numel()
    Tq = rows // B
    HI, dI = p.shape[-2], p.shape[-1]
    if idx is None:
        idx = torch.empty((rows, k), dtype=torch.int32, device=p.device)
    check(lib.lca_csa_index_topk(_ptr(p), _ptr(omega), _ptr(ikey), _ptr(csa_off), _ptr(q_pos), B, Tq, HI, dI, k, m,
                                 w, int(max_entries), _ptr(idx), _ptr(scores), _ptr(ws), ws.numel() * ws.element_size(),
                                 _index_dtype(p, ikey), _stream()), "csa_index_topk")
    return idx


def csa_index_score(p, omega, ikey, csa_off, q_pos, k: int, m: int, w: int, max_entries: int, ws: torch.Tensor,
                    scores: Optional[torch.Tensor] = None):
    """First half of csa_index_topk (scores + selection histogram)."""
    _dev(p, omega, ikey, csa_off, q_pos, ws, scores)
    B = csa_off.numel() - 1
    rows = q_pos.numel()
    check(lib.lca_csa_index_score(_ptr(p), _ptr(omega), _ptr(ikey), _ptr(csa_off), _ptr(q_pos), B, rows // B,
                                  p.shape[-2], p.shape[-1], k, m, w, int(max_entries), _ptr(scores), _ptr(ws),
                                  ws.numel() * ws.element_size(), _index_dtype(p, ikey), _stream()), "csa_index_score")


def csa_index_score_append(p, omega, ikey, csa_off, q_pos, k: int, m: int, w: int, max_entries: int,
                           ws: torch.Tensor, idx_stream: dict, kv_streams: Sequence[dict], tok_off: torch.Tensor,
                           done_len: torch.Tensor, eps: float = 1e-6, scores: Optional[torch.Tensor] = None):
    """kv_compress of the indexer-key stream and kv_streams (entries completed
    after done_len tokens) and csa_index_score for the Tq query rows of each
    sequence (q_pos holds B * Tq positions), in one launch."""
    _dev(p, omega, ikey, csa_off, q_pos, ws, scores, tok_off, done_len)
    _i64(tok_off, "tok_off")
    _i64(done_len, "done_len")
    B = csa_off.numel() - 1
    rows = q_pos.numel()
    if rows % B:
        raise ValueError("q_pos must hold the same number of rows for every sequence")
    if len(kv_streams) > 4:
        raise ValueError("0..4 kv streams per call")
    ia, _ = _stream_array([idx_stream])
    ka, _ = _stream_array(kv_streams)
    check(lib.lca_csa_index_score_append(_ptr(p), _ptr(omega), _ptr(ikey), _ptr(csa_off), _ptr(q_pos), B,
                                         rows // B, p.shape[-2], p.shape[-1], k, m, w, int(max_entries), ia, ka,
                                         len(kv_streams), _ptr(tok_off), _ptr(done_len), float(eps), _ptr(scores),
                                         _ptr(ws), ws.numel() * ws.element_size(), _index_dtype(p, ikey), _stream()),
          "csa_index_score_append")


def decode_front(p, omega, ikey, csa_off, q_pos, k: int, m: int, w: int, max_entries: int, ws: torch.Tensor,
                 idx_stream: dict, kv_streams: Sequence[dict], tok_off: torch.Tensor, done_len: torch.Tensor,
                 q, sources: Sequence[dict], scale: float, eps: float = 1e-6,
                 scores: Optional[torch.Tensor] = None):
    """csa_index_score_append followed by hybrid_attn(q, q_pos, sources), in
    one launch where it applies: the appends, the index scores and the
    attention over dense / window sources (a dense source over a cache the
    appends write takes part 1 with this done_len).  Returns the sources'
    (o_part, lse) pairs."""
    _dev(p, omega, ikey, csa_off, q_pos, ws, scores, tok_off, done_len, q)
    _i64(tok_off, "tok_off")
    _i64(done_len, "done_len")
    B = csa_off.numel() - 1
    rows = q_pos.numel()
    if rows % B:
        raise ValueError("q_pos must hold the same number of rows for every sequence")
    if len(kv_streams) > 4:
        raise ValueError("0..4 kv streams per call")
    ia, _ = _stream_array([idx_stream])
    ka, _ = _stream_array(kv_streams)
    arr, outs, Bs = _attn_sources(q, q_pos, sources)
    if Bs != B:
        raise ValueError("the sources and the caches must hold the same sequences")
    _, H, D = q.shape
    check(lib.lca_decode_front(_ptr(p), _ptr(omega), _ptr(ikey), _ptr(csa_off), _ptr(q_pos), B, rows // B,
                               p.shape[-2], p.shape[-1], k, m, w, int(max_entries), ia, ka, len(kv_streams),
                               _ptr(tok_off), _ptr(done_len), float(eps), _ptr(scores), _ptr(ws),
                               ws.numel() * ws.element_size(), arr, len(sources), _ptr(q), H, D, float(scale),
                               _index_dtype(p, ikey), _stream()), "decode_front")
    return outs


def csa_topk_select(csa_off, q_pos, k: int, m: int, w: int, max_entries: int, ws: torch.Tensor,
                    idx: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None):
    """Second half of csa_index_topk: exact top-k from the scored workspace."""
    _dev(csa_off, q_pos, ws, idx, scores)
    B = csa_off.numel() - 1
    rows = q_pos.numel()
    if idx is None:
        idx = torch.empty((rows, k), dtype=torch.int32, device=q_pos.device)
    check(lib.lca_csa_topk_select(_ptr(csa_off), _ptr(q_pos), B, rows // B, k, m, w, int(max_entries), _ptr(idx),
                                  _ptr(scores), _ptr(ws), ws.numel() * ws.element_size(), _stream()),
          "csa_topk_select")
    return idx


# ---------------------------------------------------------------- attention partials

def _parts_out(rows, H, D, n_split, device, o_part, lse, half=False):
    """Partial buffers: o_part fp32, or fp16 (half: the fp16 partials of the
    matrix-core decode kernel); lse fp32."""
    if o_part is None:
        o_part = torch.empty((n_split, rows, H, D), dtype=torch.float16 if half else torch.float32, device=device)
    if o_part.dtype not in (torch.float32, torch.float16):
        raise TypeError("o_part must be float32 or float16")
    if lse is None:
        lse = torch.empty((n_split, rows, H), dtype=torch.float32, device=device)
    return o_part, lse


def csa_sparse_attn(q, kv_csa, csa_off, idx, scale: float, eps: float, n_split: int,
                    o_part=None, lse=None):
    """q [B*Tq, H, D] raw; idx int32 [B*Tq, k].  Returns (o_part, lse)."""
    _dev(q, kv_csa, csa_off, idx, o_part, lse)
    _i64(csa_off, "csa_off")
    _i32(idx, "idx")
    B = csa_off.numel() - 1
    rows, H, D = q.shape
    Tq = rows // B
    k = idx.shape[-1]
    o_part, lse = _parts_out(rows, H, D, n_split, q.device, o_part, lse)
    check(lib.lca_csa_sparse_attn(_ptr(q), _ptr(kv_csa), _ptr(csa_off), _ptr(idx), B, Tq, H, D, k, float(scale),
                                  float(eps), n_split, _ptr(o_part), _ptr(lse), _dtype_code(q), _stream()),
          "csa_sparse_attn")
    return o_part, lse


def hca_attn(q, kv_hca, hca_off, q_pos, m2: int, w2: int, max_entries: int, scale: float, eps: float,
             n_split: int, o_part=None, lse=None):
    _dev(q, kv_hca, hca_off, q_pos, o_part, lse)
    _i64(hca_off, "hca_off")
    _i32(q_pos, "q_pos")
    B = hca_off.numel() - 1
    rows, H, D = q.shape
    Tq = rows // B
    o_part, lse = _parts_out(rows, H, D, n_split, q.device, o_part, lse)
    check(lib.lca_hca_attn(_ptr(q), _ptr(kv_hca), _ptr(hca_off), _ptr(q_pos), B, Tq, H, D, m2, w2, int(max_entries),
                           float(scale), float(eps), n_split, _ptr(o_part), _ptr(lse), _dtype_code(q), _stream()),
          "hca_attn")
    return o_part, lse


# ---------------------------------------------------------------- window + sink + merge

def swa_attn(q, x, tok_off, q_pos, W: int, scale: float, eps: float, o_part=None, lse=None):
    """The window branch as a one-split partial (o_part [1, rows, H, D], lse)."""
    _dev(q, x, tok_off, q_pos, o_part, lse)
    _i64(tok_off, "tok_off")
    _i32(q_pos, "q_pos")
    B = tok_off.numel() - 1
    rows, H, D = q.shape
    o_part, lse = _parts_out(rows, H, D, 1, q.device, o_part, lse)
    check(lib.lca_swa_attn(_ptr(q), _ptr(x), _ptr(tok_off), _ptr(q_pos), B, rows // B, H, D, W, float(scale),
                           float(eps), _ptr(o_part), _ptr(lse), _dtype_code(q), _stream()), "swa_attn")
    return o_part, lse


_KINDS = {"dense": LCA_SRC_DENSE, "gather": LCA_SRC_GATHER, "window": LCA_SRC_WINDOW, "topk": LCA_SRC_TOPK}


def _attn_sources(q, q_pos, sources: Sequence[dict]):
    """ctypes array of the sources, their (o_part, lse) outputs and B."""
    if not 1 <= len(sources) <= 3:
        raise ValueError("1..3 sources per call")
    _dev(q, q_pos)
    if q_pos is not None:
        _i32(q_pos, "q_pos")
    rows, H, D = q.shape
    arr = (AttnSource * len(sources))()
    outs = []
    B = None
    for i, s in enumerate(sources):
        kind = _KINDS[s["kind"]]
        kv, off, idx = s["kv"], s["off"], s.get("idx")
        _dev(kv, off, idx)
        _i64(off, "off")
        if B is None:
            B = off.numel() - 1
        elif off.numel() - 1 != B:
            raise ValueError("every source needs the same number of sequences")
        k = 0
        ws = ws_bytes = max_entries = scores = idx_out = None
        if kind == LCA_SRC_GATHER:
            _i32(idx, "idx")
            k = idx.shape[-1]
        if kind == LCA_SRC_TOPK:
            idx_out, ws, scores = s["idx_out"], s["ws"], s.get("scores")
            _dev(idx_out, ws, scores)
            _i32(idx_out, "idx_out")
            k = int(s["k"])
            if idx_out.shape != (rows, k):
                raise ValueError(f"idx_out must be [{rows}, {k}]")
            ws_bytes, max_entries = ws.numel() * ws.element_size(), int(s["max_entries"])
        ns = int(s["n_split"])
        o_part, lse = _parts_out(rows, H, D, ns, q.device, s.get("o_part"), s.get("lse"), bool(s.get("o_half")))
        _dev(o_part, lse)
        done_len, part = s.get("done_len"), int(s.get("part", 0))
        if part:
            _dev(done_len)
            _i64(done_len, "done_len")
        v = s.get("v")
        if v is not None:
            _dev(v)
            if v.shape != kv.shape or v.dtype != kv.dtype:
                raise TypeError("values shaped and typed as the keys")
        arr[i] = AttnSource(kind, kv.data_ptr(), off.data_ptr(), None if idx is None else idx.data_ptr(), k,
                            int(s.get("m2", 1)), int(s.get("w2", 1)), int(s.get("W", 0)), ns, o_part.data_ptr(),
                            lse.data_ptr(), _addr(ws), ws_bytes or 0, max_entries or 0, _addr(scores), _addr(idx_out),
                            _addr(done_len) if part else None, part, int(s.get("rope", 0)),
                            float(s.get("rope_base", 10000.0)), int(s.get("tiles_per_split", 0)), _addr(v),
                            int(o_part.dtype == torch.float16))
        outs.append((o_part, lse))
    return arr, outs, B


def hybrid_attn(q, q_pos, sources: Sequence[dict], scale: float, eps: float):
    """The attention branches of a step in one launch.  sources: dicts with
    kind ("gather", "dense", "window" or "topk"), kv, off and n_split, plus
    idx (gather), m2 and w2 (dense), W (window), and optionally o_part / lse,
    tiles_per_split (a fixed partition of each row's keys), rope / rope_base
    (the rotary embedding of the call: the same in every source), o_half
    (fp16 partials, allocated when o_part is not given; a given o_part's
    dtype, float32 or float16, decides) and, for a dense
    source, part (1: the entries complete within the first done_len[b]
    tokens; 2: those completed after them) with done_len (int64 [B]).
    A "topk" source selects the sparse branch's entries from the scores a
    csa_index_score(_append) call left in its workspace: it takes k, m2 = m,
    w2 = w, max_entries, ws, idx_out (int32 [rows, k], written) and
    optionally scores.  Returns one (o_part, lse) pair per source, as the
    single-branch calls."""
    arr, outs, B = _attn_sources(q, q_pos, sources)
    rows, H, D = q.shape
    check(lib.lca_hybrid_attn(arr, len(sources), _ptr(q), _ptr(q_pos), B, rows // B, H, D, float(scale), float(eps),
                              _dtype_code(q), _stream()), "hybrid_attn")
    return outs


def hybrid_attn_merge(q, q_pos, sources: Sequence[dict], sigma, scale: float, eps: float, out=None):
    """The sources of hybrid_attn merged with the sink sigma (fp32 [H] or
    None) into out [rows, H, D] (q's dtype), as hybrid_attn + swa_merge; one
    launch on the row-tiled path with one split per source (the partial
    buffers are then not written).  Returns out."""
    arr, _, B = _attn_sources(q, q_pos, sources)
    _dev(sigma, out)
    rows, H, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    check(lib.lca_hybrid_attn_merge(arr, len(sources), _ptr(q), _ptr(q_pos), B, rows // B, H, D, float(scale),
                                    float(eps), _ptr(sigma), _ptr(out), _dtype_code(q), _stream()),
          "hybrid_attn_merge")
    return out


def swa_merge_workspace(n_rows: int, H: int, D: int) -> int:
    return int(lib.lca_swa_merge_workspace(n_rows, H, D))


def swa_merge(q, x, tok_off, q_pos, sink, parts, W: int, scale: float, eps: float, ws: torch.Tensor,
              out=None):
    """parts: list of (o_part, lse) pairs (o_part float32 or float16).
    Returns out [B*Tq, H, D] (q's dtype).
    With W = 0 only the partials and the sink are merged (x, tok_off, q_pos
    and ws may be None)."""
    _dev(q, x, tok_off, q_pos, sink, ws, out)
    rows, H, D = q.shape
    if W > 0:
        _i64(tok_off, "tok_off")
        _i32(q_pos, "q_pos")
        B = tok_off.numel() - 1
        Tq = rows // B
    else:
        B, Tq = rows, 1
    arr = (Partial * max(1, len(parts)))()
    for i, (o, l) in enumerate(parts):
        _dev(o, l)
        if o.dtype not in (torch.float32, torch.float16):
            raise TypeError("partials must be float32 or float16")
        arr[i] = Partial(o.data_ptr(), l.data_ptr(), o.shape[0], int(o.dtype == torch.float16))
    if out is None:
        out = torch.empty_like(q)
    if sink is not None and sink.dtype != torch.float32:
        raise TypeError("sink must be float32")
    check(lib.lca_swa_merge(_ptr(q), _ptr(x), _ptr(tok_off), _ptr(q_pos), _ptr(sink), arr, len(parts), B, Tq, H, D,
                            W, float(scale), float(eps), _ptr(out), _ptr(ws),
                            0 if ws is None else ws.numel() * ws.element_size(), _dtype_code(q), _stream()),
          "swa_merge")
    return out
