"""Seeded synthetic inputs for the hybrid compressed attention hot path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the CPU oracle tests and the GPU path (tests, bench)
take their inputs from here, so that the two sides see identical bits.

Workloads follow the shapes that the DeepSeek-V4 pages give for the attention
stack ("DeepSeek-V4" spec sheet, Per-variant configs and Core block; "Why
DeepSeek V4 Stands Apart", Core Architectural Innovations):

* ``tiny``           1 x 4096 tokens, 4 heads x 64, indexer 2 x 32, top-64, fp32
* ``flash_decode``   8 x 131072 tokens, 64 heads x 512, indexer 4 x 64, top-512
* ``pro_1m_decode``  1 x 1048576 tokens, 128 heads x 512, indexer 4 x 64, top-1024
* ``flash_prefill``  4096 new tokens after 262144 cached, 64 heads x 512, top-512
* ``pro_varlen``     64 sequences, lengths uniform on [16384, 262144], 128 x 512,
                     top-1024, 32 planted high-norm indexer-key runs per sequence

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence([cfg_id,
layer, tensor_id]))`` as float32 N(0, 1) and then rounded to bfloat16
(round-to-nearest-even) for the bf16 workloads.  Large workloads can instead be
drawn on the GPU with a seeded ``torch.Generator`` (``make_raw_torch``), which
is much faster; the oracle then reads those values back from the device.

Tensor ids: x=0 (raw KV), a=1 (CSA pooling logits), g=2 (HCA pooling logits),
u=3 (raw indexer keys), c=4 (indexer pooling logits), q=5, p=6 (indexer
queries), omega=7 (indexer head weights), sigma=8 (sink logits), lens=9,
plant=10; with the dual-stream compressor the second-half streams x_b=11,
a_b=12, u_b=13, c_b=14; with separate values the raw value tokens v=15 (and
v_b=16 with both options).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

TID = dict(x=0, a=1, g=2, u=3, c=4, q=5, p=6, omega=7, sigma=8, lens=9, plant=10, x_b=11, a_b=12, u_b=13, c_b=14,
           v=15, v_b=16)


@dataclass(frozen=True)
class Config:
    """Shape of one workload.  ``lens`` are the context lengths per sequence
    (for prefill: the total length after the chunk); ``tq`` is the number of
    query tokens per sequence (the last ``tq`` positions)."""

    name: str
    cfg_id: int
    B: int
    lens: Tuple[int, ...]
    tq: int
    H: int
    D: int
    HI: int
    dI: int
    k: int
    dtype: str  # "bf16" or "f32"
    m: int = 4
    w: int = 8
    m2: int = 128
    w2: int = 128
    W: int = 128
    plant: int = 0
    eps: float = 1e-6
    logit_per_channel: bool = True
    ikey: str = "bf16"  # indexer-key cache: "bf16" (the workload dtype), "fp8" (E4M3 rows with a scale) or "mxfp4"
    rope: int = 0       # rotated dims at the end of each head (0: no rotary embedding)
    rope_base: float = 10000.0
    dual: bool = False  # CSA windows: first half from (x, a) / (u, c), second half from (x_b, a_b) / (u_b, c_b)
    sepv: bool = False  # values from their own raw stream v (keys from x)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def _varlen_lengths(cfg_id: int, B: int, lo: int, hi: int, layer: int = 0) -> Tuple[int, ...]:
    r = rng_for(cfg_id, layer, TID["lens"])
    return tuple(int(v) for v in r.integers(lo, hi, size=B, endpoint=True))


def rng_for(cfg_id: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, layer, tensor_id]))


TINY = Config("tiny", 0, 1, (4096,), 1, 4, 64, 2, 32, 64, "f32")
FLASH_DECODE = Config("flash_decode", 1, 8, (131072,) * 8, 1, 64, 512, 4, 64, 512, "bf16")
PRO_1M_DECODE = Config("pro_1m_decode", 2, 1, (1048576,), 1, 128, 512, 4, 64, 1024, "bf16")
FLASH_PREFILL = Config("flash_prefill", 3, 1, (262144 + 4096,), 4096, 64, 512, 4, 64, 512, "bf16")
PRO_VARLEN = Config("pro_varlen", 4, 64, _varlen_lengths(4, 64, 16384, 262144), 1, 128, 512, 4, 64,
                    1024, "bf16", plant=32)

# The Pro 1M decode with two query rows per step (the main token and one
# drafted by the multi-token-prediction module, verified together).
PRO_1M_MTP2 = Config("pro_1m_mtp2", 5, 1, (1048576,), 2, 128, 512, 4, 64, 1024, "bf16")

# The Pro 1M decode (same seeds) with the indexer-key cache as fp8 rows.
PRO_1M_DECODE_FP8 = dataclasses.replace(PRO_1M_DECODE, name="pro_1m_decode_fp8", ikey="fp8")
# The Pro variable-length batch decode (same seeds) with fp8 indexer keys.
PRO_VARLEN_FP8 = dataclasses.replace(PRO_VARLEN, name="pro_varlen_fp8", ikey="fp8")
# The Pro 1M decode (same seeds) with MXFP4 indexer keys.
PRO_1M_DECODE_MXFP4 = dataclasses.replace(PRO_1M_DECODE, name="pro_1m_decode_mxfp4", ikey="mxfp4")
# The Flash prefill chunk (same seeds) with fp8 indexer keys.
FLASH_PREFILL_FP8 = dataclasses.replace(FLASH_PREFILL, name="flash_prefill_fp8", ikey="fp8")
# The Pro variable-length batch and the Flash prefill chunk (same seeds) with
# MXFP4 indexer keys.
PRO_VARLEN_MXFP4 = dataclasses.replace(PRO_VARLEN, name="pro_varlen_mxfp4", ikey="mxfp4")
FLASH_PREFILL_MXFP4 = dataclasses.replace(FLASH_PREFILL, name="flash_prefill_mxfp4", ikey="mxfp4")

# The Pro 1M decode (same seeds) with the partial rotary embedding on the
# last 64 dims of each head; and with every model option at once: the rotary
# embedding, the dual-stream compressor and separate values.
PRO_1M_DECODE_ROPE = dataclasses.replace(PRO_1M_DECODE, name="pro_1m_decode_rope", rope=64)
PRO_1M_DECODE_ALL = dataclasses.replace(PRO_1M_DECODE, name="pro_1m_decode_all_options", rope=64, dual=True,
                                        sepv=True)

CONFIGS: Dict[str, Config] = {c.name: c for c in (TINY, FLASH_DECODE, PRO_1M_DECODE, FLASH_PREFILL, PRO_VARLEN,
                                                  PRO_1M_MTP2, PRO_1M_DECODE_FP8, PRO_VARLEN_FP8, FLASH_PREFILL_FP8,
                                                  PRO_1M_DECODE_MXFP4, PRO_VARLEN_MXFP4, FLASH_PREFILL_MXFP4,
                                                  PRO_1M_DECODE_ROPE, PRO_1M_DECODE_ALL)}


def small(name: str, cfg_id: int, lens, tq: int = 1, H: int = 64, D: int = 512, HI: int = 4,
          dI: int = 64, k: int = 512, dtype: str = "bf16", **kw) -> Config:
    """A cut-down workload with the same structure (used by the parity tests)."""
    return Config(name, cfg_id, len(lens), tuple(int(v) for v in lens), tq, H, D, HI, dI, k, dtype, **kw)


# ----------------------------------------------------------------------------
# rounding used to *store* generated values (not part of the method)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize(x: np.ndarray, dtype: str) -> np.ndarray:
    """Return float32 values representable in ``dtype``."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def _normal(cfg: Config, layer: int, tid: int, shape, dtype: str) -> np.ndarray:
    r = rng_for(cfg.cfg_id, layer, tid)
    return quantize(r.standard_normal(size=shape, dtype=np.float32), dtype)


def offsets(lens) -> np.ndarray:
    o = np.zeros(len(lens) + 1, dtype=np.int64)
    o[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return o


def plant_positions(cfg: Config, layer: int, b: int, n_csa: int) -> np.ndarray:
    """Start tokens (multiples of m) of the planted indexer-key runs of sequence b."""
    if cfg.plant <= 0 or n_csa <= 0:
        return np.zeros(0, dtype=np.int64)
    r = rng_for(cfg.cfg_id, layer, TID["plant"] * 1000 + b)
    ent = np.sort(r.choice(n_csa, size=min(cfg.plant, n_csa), replace=False))
    return ent.astype(np.int64) * cfg.m


def plant_vector(cfg: Config, layer: int) -> np.ndarray:
    """One seeded direction shared by all planted runs, with norm 8*sqrt(dI)."""
    r = rng_for(cfg.cfg_id, layer, TID["plant"])
    v = r.standard_normal(cfg.dI).astype(np.float64)
    v = v / np.linalg.norm(v) * 8.0 * np.sqrt(cfg.dI)
    return quantize(v.astype(np.float32), cfg.dtype)


def _n_full_windows(L: int, m: int, w: int) -> int:
    # number of complete windows of length w at stride m (used only to place
    # the planted runs inside the stream)
    return 0 if L < w else (L - w) // m + 1


def make_raw(cfg: Config, layer: int = 0) -> Dict[str, np.ndarray]:
    """Host (numpy) inputs.  Raw streams are packed over sequences."""
    T = int(sum(cfg.lens))
    dt = cfg.dtype
    out: Dict[str, np.ndarray] = {}
    out["tok_off"] = offsets(cfg.lens)
    out["x"] = _normal(cfg, layer, TID["x"], (T, cfg.D), dt)
    lshape_kv = (T, cfg.D) if cfg.logit_per_channel else (T,)
    lshape_i = (T, cfg.dI) if cfg.logit_per_channel else (T,)
    out["a"] = _normal(cfg, layer, TID["a"], lshape_kv, dt)
    out["g"] = _normal(cfg, layer, TID["g"], lshape_kv, dt)
    out["u"] = _normal(cfg, layer, TID["u"], (T, cfg.dI), dt)
    out["c"] = _normal(cfg, layer, TID["c"], lshape_i, dt)
    Q = cfg.B * cfg.tq
    out["q"] = _normal(cfg, layer, TID["q"], (Q, cfg.H, cfg.D), dt)
    out["p"] = _normal(cfg, layer, TID["p"], (Q, cfg.HI, cfg.dI), dt)
    out["omega"] = _normal(cfg, layer, TID["omega"], (Q, cfg.HI), "f32")
    out["sigma"] = _normal(cfg, layer, TID["sigma"], (cfg.H,), "f32")
    for name, shape in _option_streams(cfg, T):
        out[name] = _normal(cfg, layer, TID[name], shape, dt)
    q_pos = np.zeros((cfg.B, cfg.tq), dtype=np.int32)
    for b, L in enumerate(cfg.lens):
        q_pos[b] = np.arange(L - cfg.tq, L, dtype=np.int32)
    out["q_pos"] = q_pos
    if cfg.plant > 0:
        v = plant_vector(cfg, layer)
        for b, L in enumerate(cfg.lens):
            base = int(out["tok_off"][b])
            for t0 in plant_positions(cfg, layer, b, _n_full_windows(L, cfg.m, cfg.w)):
                out["u"][base + t0: base + t0 + cfg.w] = v[None, :]
                if cfg.dual:
                    out["u_b"][base + t0: base + t0 + cfg.w] = v[None, :]
    return out


def _option_streams(cfg: Config, T: int):
    """(name, shape) of the raw streams the dual-stream compressor and the
    separate values add."""
    lshape_kv = (T, cfg.D) if cfg.logit_per_channel else (T,)
    lshape_i = (T, cfg.dI) if cfg.logit_per_channel else (T,)
    out = []
    if cfg.dual:
        out += [("x_b", (T, cfg.D)), ("a_b", lshape_kv), ("u_b", (T, cfg.dI)), ("c_b", lshape_i)]
    if cfg.sepv:
        out.append(("v", (T, cfg.D)))
        if cfg.dual:
            out.append(("v_b", (T, cfg.D)))
    return out


def make_raw_torch(cfg: Config, layer: int = 0, device: str = "cuda"):
    """Device-side inputs drawn with a seeded torch.Generator (fast for the
    million-token workloads).  Same layout and distributions as ``make_raw``;
    different bits.  Returns a dict of torch tensors."""
    import torch

    T = int(sum(cfg.lens))
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def normal(tid, shape, dtype=tdt):
        gen = torch.Generator(device=device)
        gen.manual_seed(int(np.random.SeedSequence([cfg.cfg_id, layer, tid, 7]).generate_state(1)[0]))
        t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        return t.to(dtype)

    out = {}
    out["tok_off"] = torch.from_numpy(offsets(cfg.lens)).to(device)
    out["x"] = normal(TID["x"], (T, cfg.D))
    lshape_kv = (T, cfg.D) if cfg.logit_per_channel else (T,)
    lshape_i = (T, cfg.dI) if cfg.logit_per_channel else (T,)
    out["a"] = normal(TID["a"], lshape_kv)
    out["g"] = normal(TID["g"], lshape_kv)
    out["u"] = normal(TID["u"], (T, cfg.dI))
    out["c"] = normal(TID["c"], lshape_i)
    Q = cfg.B * cfg.tq
    out["q"] = normal(TID["q"], (Q, cfg.H, cfg.D))
    out["p"] = normal(TID["p"], (Q, cfg.HI, cfg.dI))
    out["omega"] = normal(TID["omega"], (Q, cfg.HI), torch.float32)
    out["sigma"] = normal(TID["sigma"], (cfg.H,), torch.float32)
    for name, shape in _option_streams(cfg, T):
        out[name] = normal(TID[name], shape)
    q_pos = np.zeros((cfg.B, cfg.tq), dtype=np.int32)
    for b, L in enumerate(cfg.lens):
        q_pos[b] = np.arange(L - cfg.tq, L, dtype=np.int32)
    out["q_pos"] = torch.from_numpy(q_pos).to(device)
    if cfg.plant > 0:
        v = torch.from_numpy(plant_vector(cfg, layer)).to(device=device, dtype=tdt)
        offs = offsets(cfg.lens)
        for b, L in enumerate(cfg.lens):
            pos = plant_positions(cfg, layer, b, _n_full_windows(L, cfg.m, cfg.w))
            if len(pos) == 0:
                continue
            rows = (torch.from_numpy(pos)[:, None] + torch.arange(cfg.w)[None, :]).reshape(-1) + int(offs[b])
            out["u"][rows.to(device)] = v
            if cfg.dual:
                out["u_b"][rows.to(device)] = v
    return out
