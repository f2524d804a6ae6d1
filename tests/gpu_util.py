"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
HIP path through the C-ABI, and compare against the oracle."""
import numpy as np
import torch

import lca_inputs as li
from oracle import attention as oatt
from oracle import indexer as oidx
from oracle import pipeline as opipe

TOL = {"bf16": 2e-2, "f32": 1e-4}     # max-abs output tolerance
REL = {"bf16": 1e-2, "f32": 1e-5}     # extra: relative Frobenius error
U32 = 2.0 ** -24


def tdtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def to_device(raw, cfg, dev="cuda"):
    dt = tdtype(cfg)
    d = {}
    for k in ("x", "a", "g", "u", "c", "q", "p") + opipe.OPTION_STREAMS:
        if k in raw:
            d[k] = torch.from_numpy(np.ascontiguousarray(raw[k])).to(dev).to(dt)
    d["omega"] = torch.from_numpy(raw["omega"]).to(dev).contiguous()
    d["sigma"] = torch.from_numpy(raw["sigma"]).to(dev).contiguous()
    d["tok_off"] = torch.from_numpy(raw["tok_off"]).to(dev)
    d["q_pos"] = torch.from_numpy(np.ascontiguousarray(raw["q_pos"].reshape(-1))).to(dev)
    return d


def layer_for(cfg, **kw):
    from long_context_attention_20_amd import HybridAttention
    kw.setdefault("ikey", getattr(cfg, "ikey", "bf16"))
    kw.setdefault("rope", getattr(cfg, "rope", 0))
    kw.setdefault("rope_base", getattr(cfg, "rope_base", 10000.0))
    kw.setdefault("dual", getattr(cfg, "dual", False))
    kw.setdefault("sepv", getattr(cfg, "sepv", False))
    return HybridAttention(cfg.H, cfg.D, cfg.HI, cfg.dI, cfg.k, cfg.m, cfg.w, cfg.m2, cfg.w2, cfg.W, cfg.eps, **kw)


def fp8_rows(t):
    """An fp8 key cache (uint8 rows: d_I E4M3 bytes, fp32 scale, 4 zero bytes)
    -> (q [N, d_I] float64 E4M3 values, s [N] float64 scales, pad [N, 4])."""
    t = t.contiguous().cpu()
    dI = t.shape[1] - 8
    q = t[:, :dI].contiguous().view(torch.float8_e4m3fn).to(torch.float64).numpy()
    s = t[:, dI:dI + 4].contiguous().view(torch.float32).to(torch.float64).numpy()[:, 0]
    return q, s, t[:, dI + 4:].numpy()


E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def mx_rows(t, dI):
    """An MXFP4 key cache (uint8 rows: d_I/2 bytes of E2M1 pairs, the even
    channel in the low nibble, then d_I/32 E8M0 scale bytes, zero pad) ->
    (q [N, d_I] E2M1 values, s [N, d_I/32] scales, pad bytes)."""
    t = t.contiguous().cpu().numpy()
    b = t[:, :dI // 2]
    nib = np.stack([b & 15, b >> 4], axis=-1).reshape(t.shape[0], dI)
    q = E2M1_VALUES[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    codes = t[:, dI // 2:dI // 2 + dI // 32].astype(np.int64)
    s = np.where(codes > 0, np.ldexp(1.0, codes - 127), 2.0 ** -127)
    return q, s, t[:, dI // 2 + dI // 32:]


def key_rows(ikey, dI=None):
    """The indexer-key rows a cache stands for (float64): bf16/fp32 rows as
    they are, fp8 rows as scale * value, MXFP4 rows as block scale * value
    (dI tells the two byte layouts apart)."""
    if ikey.dtype == torch.uint8:
        if dI is not None and ikey.shape[1] == dI // 2 + 8:
            q, s, _ = mx_rows(ikey, dI)
            return (q.reshape(q.shape[0], -1, 32) * s[..., None]).reshape(q.shape)
        q, s, _ = fp8_rows(ikey)
        return q * s[:, None]
    return f64(ikey)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def seq_caches(caches, b):
    co, ho = caches.csa_off_h, caches.hca_off_h
    vals = getattr(caches, "v_csa", None) is not None
    return opipe.SeqCaches(f64(caches.kv_csa[co[b]:co[b + 1]]), f64(caches.ikey[co[b]:co[b + 1]]),
                           f64(caches.kv_hca[ho[b]:ho[b + 1]]),
                           f64(caches.v_csa[co[b]:co[b + 1]]) if vals else None,
                           f64(caches.v_hca[ho[b]:ho[b + 1]]) if vals else None)


def run_gpu(cfg, raw, dev="cuda", mode="A", **kw):
    d = to_device(raw, cfg, dev)
    layer = layer_for(cfg, **kw)
    caches = layer.alloc_caches(cfg.lens, dev, tdtype(cfg))
    layer.compress(caches, d, d["tok_off"])
    out, inter = layer.step(caches, d["x"], d["tok_off"], d["q"], d["p"], d["omega"], d["sigma"], d["q_pos"],
                            raw["q_pos"].reshape(-1), mode=mode, keep=True, v=d.get("v"))
    torch.cuda.synchronize()
    return d, layer, caches, out, inter


def merge_splits(o_part, lse):
    """GPU split partials of one row -> (o [H, D], lse [H]) via the oracle merge."""
    parts = [(f64(o_part[s]), f64(lse[s])) for s in range(o_part.shape[0])]
    return oatt.merge(parts, None)


def score_bound(p, omega, keys):
    """A-priori bound on |fp32 score - exact score| for every key."""
    p = np.asarray(p, np.float64)
    om = np.abs(np.asarray(omega, np.float64))
    mag = np.abs(keys) @ np.abs(p).T            # [N, HI]
    n = p.shape[1] + p.shape[0] + 4
    return 2.0 * n * U32 * (mag @ om) + 1e-30


def check_topk(sel_gpu, s_gpu, s_ref, bound, k):
    """Set checks for one query row.  Returns the number of accepted near-tie
    differences."""
    nv = len(s_ref)
    sel = np.asarray(sel_gpu)
    assert np.all(sel[sel >= 0] < nv), "selected an invisible entry"
    chosen = sel[sel >= 0]
    assert len(set(chosen.tolist())) == len(chosen), "duplicate index"
    if nv <= k:
        assert sorted(chosen.tolist()) == list(range(nv))
        assert np.all(sel[nv:] == -1)
        return 0
    assert len(chosen) == k
    # exact self-consistency with the GPU's own fp32 scores
    self_ref = set(oidx.topk(np.asarray(s_gpu[:nv], np.float64), k).tolist())
    assert set(chosen.tolist()) == self_ref, "selection is not the exact top-k of the GPU scores"
    # GPU scores against the oracle
    err = np.abs(np.asarray(s_gpu[:nv], np.float64) - s_ref)
    assert np.all(err <= bound), f"score error {np.max(err / bound):.2f}x the fp32 bound"
    ref = oidx.topk(s_ref, k)
    kth = s_ref[ref[-1]]
    diff = set(chosen.tolist()) ^ set(ref.tolist())
    for j in diff:
        assert abs(s_ref[j] - kth) <= 1e-6 * max(1.0, abs(kth)) + bound[j], \
            f"entry {j}: score {s_ref[j]} vs k-th {kth}: not a tie"
    return len(diff)


def assert_close(got, ref, dtype, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.max(np.abs(got - ref)) if got.size else 0.0
    assert err <= TOL[dtype], f"{what}: max-abs {err:.3e} > {TOL[dtype]}"
    nrm = np.linalg.norm(ref)
    if nrm > 0:
        rel = np.linalg.norm(got - ref) / nrm
        assert rel <= REL[dtype], f"{what}: relative error {rel:.3e} > {REL[dtype]}"
    return err
