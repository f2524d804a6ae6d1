"""ctypes view of liblca.so (the C-ABI declared in include/lca.h).

The library must have been built (``python -m long_context_attention_20_amd.build``);
there is no fallback: loading fails loudly when it is missing.
"""
import ctypes
import os

# torch first: torch ships its own HIP runtime with the same soname as the
# system one; loading it first makes liblca bind to that single runtime.
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblca.so")

LCA_OK = 0
LCA_ERR_INVALID_ARG = -1
LCA_ERR_UNSUPPORTED = -2
LCA_ERR_WORKSPACE = -3
LCA_ERR_HIP = -4
LCA_F32 = 0
LCA_BF16 = 1
LCA_BF16_FP8KEY = 2  # index calls: bf16 queries, fp8 key rows (d_I E4M3 bytes, fp32 scale, 4 zero bytes)
LCA_BF16_MXFP4KEY = 3  # index calls: bf16 queries, MXFP4 key rows (d_I/2 bytes of E2M1 pairs, E8M0 scales, pad)

EXPORTS = [
    "lca_strerror", "lca_last_error", "lca_version", "lca_kv_compress",
    "lca_csa_index_topk_workspace", "lca_csa_index_topk", "lca_csa_index_score", "lca_csa_index_score_append",
    "lca_csa_topk_select", "lca_csa_sparse_attn", "lca_hca_attn",
    "lca_swa_attn", "lca_hybrid_attn", "lca_swa_merge_workspace", "lca_swa_merge", "lca_hybrid_attn_merge",
    "lca_diag_trace", "lca_diag_topk_wait", "lca_decode_front",
    "lca_csa_index_topk_noalloc_max_bytes", "lca_csa_index_topk_noalloc",
]
LCA_SRC_DENSE, LCA_SRC_GATHER, LCA_SRC_WINDOW, LCA_SRC_TOPK = 0, 1, 2, 3


class CompressStream(ctypes.Structure):
    _fields_ = [
        ("src", ctypes.c_void_p), ("logits", ctypes.c_void_p), ("out", ctypes.c_void_p),
        ("ent_off", ctypes.c_void_p), ("C", ctypes.c_int32), ("m", ctypes.c_int32), ("w", ctypes.c_int32),
        ("per_channel", ctypes.c_int32), ("rmsnorm", ctypes.c_int32), ("max_entries", ctypes.c_int32),
        ("out_key", ctypes.c_int32), ("rope_dims", ctypes.c_int32), ("rope_base", ctypes.c_float),
        ("src2", ctypes.c_void_p), ("logits2", ctypes.c_void_p),
    ]


class Partial(ctypes.Structure):
    _fields_ = [("o", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("n_split", ctypes.c_int32),
                ("o_half", ctypes.c_int32)]


class AttnSource(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("kv", ctypes.c_void_p), ("off", ctypes.c_void_p), ("idx", ctypes.c_void_p),
        ("k", ctypes.c_int32), ("m2", ctypes.c_int32), ("w2", ctypes.c_int32), ("W", ctypes.c_int32),
        ("n_split", ctypes.c_int32), ("o_part", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t), ("max_entries", ctypes.c_int64),
        ("scores", ctypes.c_void_p), ("idx_out", ctypes.c_void_p),
        ("done_len", ctypes.c_void_p), ("part", ctypes.c_int32), ("rope_dims", ctypes.c_int32),
        ("rope_base", ctypes.c_float), ("tiles_per_split", ctypes.c_int32), ("v", ctypes.c_void_p),
        ("o_half", ctypes.c_int32),
    ]


class LCAError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__(f"{what}: {lib.lca_strerror(code).decode()} ({code}): {lib.lca_last_error().decode()}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python long_context_attention_20_amd/build.py` "
                          "(the HIP library is required; there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.lca_strerror.restype = ctypes.c_char_p
    L.lca_strerror.argtypes = [i32]
    L.lca_last_error.restype = ctypes.c_char_p
    L.lca_last_error.argtypes = []
    L.lca_version.restype = i32
    L.lca_kv_compress.restype = i32
    L.lca_kv_compress.argtypes = [ctypes.POINTER(CompressStream), i32, vp, vp, i32, f32, i32, vp]
    L.lca_csa_index_topk_workspace.restype = sz
    L.lca_csa_index_topk_workspace.argtypes = [i32, i64, i32]
    L.lca_csa_index_topk.restype = i32
    L.lca_csa_index_topk.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i64, vp, vp, vp, sz,
                                     i32, vp]
    L.lca_csa_index_score.restype = i32
    L.lca_csa_index_score.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i64, vp, vp, sz, i32, vp]
    L.lca_csa_index_score_append.restype = i32
    L.lca_csa_index_score_append.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i64,
                                             ctypes.POINTER(CompressStream), ctypes.POINTER(CompressStream), i32,
                                             vp, vp, f32, vp, vp, sz, i32, vp]
    L.lca_csa_topk_select.restype = i32
    L.lca_csa_topk_select.argtypes = [vp, vp, i32, i32, i32, i32, i32, i64, vp, vp, vp, sz, vp]
    L.lca_csa_sparse_attn.restype = i32
    L.lca_csa_sparse_attn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, f32, i32, vp, vp, i32, vp]
    L.lca_hca_attn.restype = i32
    L.lca_hca_attn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64, f32, f32, i32, vp, vp, i32, vp]
    L.lca_swa_attn.restype = i32
    L.lca_swa_attn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, f32, vp, vp, i32, vp]
    L.lca_hybrid_attn.restype = i32
    L.lca_hybrid_attn.argtypes = [ctypes.POINTER(AttnSource), i32, vp, vp, i32, i32, i32, i32, f32, f32, i32, vp]
    L.lca_swa_merge_workspace.restype = sz
    L.lca_swa_merge_workspace.argtypes = [i32, i32, i32]
    L.lca_swa_merge.restype = i32
    L.lca_swa_merge.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(Partial), i32, i32, i32, i32, i32, i32, f32, f32,
                                vp, vp, sz, i32, vp]
    L.lca_hybrid_attn_merge.restype = i32
    L.lca_hybrid_attn_merge.argtypes = [ctypes.POINTER(AttnSource), i32, vp, vp, i32, i32, i32, i32, f32, f32, vp, vp,
                                        i32, vp]
    L.lca_decode_front.restype = i32
    L.lca_decode_front.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i64,
                                   ctypes.POINTER(CompressStream), ctypes.POINTER(CompressStream), i32, vp, vp, f32,
                                   vp, vp, sz, ctypes.POINTER(AttnSource), i32, vp, i32, i32, f32, i32, vp]
    L.lca_csa_index_topk_noalloc_max_bytes.restype = sz
    L.lca_csa_index_topk_noalloc_max_bytes.argtypes = []
    L.lca_csa_index_topk_noalloc.restype = i32
    L.lca_csa_index_topk_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i64, vp, vp,
                                             i32, vp]
    L.lca_diag_trace.restype = i32
    L.lca_diag_trace.argtypes = [vp, i64]
    L.lca_diag_topk_wait.restype = i32
    L.lca_diag_topk_wait.argtypes = [i32, i64]
    return L


lib = _load()


def check(code: int, what: str):
    if code != LCA_OK:
        raise LCAError(code, what)
