"""fp16 attention partials (o_half): the matrix-core decode kernel stores each
split's softmax-normalised output in IEEE half precision, and both merge
kernels read it back.  Checked against the same call with fp32 partials
(per element within fp16's rounding of the fp32 value, identical lse), the
merged output against the fp32-partial merge (within bf16 rounding) and
against the oracle, and the rejection of o_half where the kernel that
would write the partials does not take it."""
import numpy as np
import pytest
import torch

import lca_inputs as li
from oracle import compress as ocmp
from oracle import pipeline as opipe

from gpu_util import assert_close, f64, layer_for, seq_caches, tdtype, to_device

pytestmark = pytest.mark.gpu

CASES = {
    # one query row per sequence, three sources with several splits (the
    # generic merge kernel)
    "pro_splits": (li.small("half_pro", 121, (9000, 5003), H=128, D=512, k=1024, plant=32), (3, 5, 1)),
    # eight sequences x 128 heads and one split per source: the merge takes
    # the per-(row, head) kernel
    "flash_rows": (li.small("half_rows", 122, (3000, 1029, 517, 7, 2600, 4100, 900, 1600), H=128, D=512, k=512),
                   (1, 1, 1)),
    # small head dim (D = 64), lengths around the window and stride edges
    "edges_h16": (li.small("half_edges", 123, (1, 7, 8, 11, 127, 128, 129, 300), H=16, D=64, HI=2, dI=32, k=8),
                  (2, 2, 1)),
}


def _half_bound(o32):
    # round to nearest even in fp16: 2^-11 of the value for normal halves,
    # 2^-25 absolute in the subnormal range
    return np.abs(o32) * 2.0 ** -11 + 2.0 ** -25


@pytest.mark.parametrize("name", sorted(CASES))
def test_half_partials_against_fp32(name):
    from long_context_attention_20_amd import ops
    cfg, (sc, sh, sw) = CASES[name]
    print(f"[half partials {name}] lens={cfg.lens} H={cfg.H} D={cfg.D} k={cfg.k} splits={sc},{sh},{sw}", flush=True)
    raw = li.make_raw(cfg)
    d = to_device(raw, cfg)
    layer = layer_for(cfg)
    caches = layer.alloc_caches(cfg.lens, "cuda", tdtype(cfg))
    layer.compress(caches, d, d["tok_off"])
    q_pos = d["q_pos"]
    qp = q_pos.cpu().numpy()
    rows = q_pos.numel()
    max_csa = max(1, ocmp.n_entries(int(qp.max()) + 1, cfg.m, cfg.w))
    idx = ops.csa_index_topk(d["p"], d["omega"], caches.ikey, caches.csa_off, q_pos, cfg.k, cfg.m, cfg.w, max_csa,
                             torch.zeros(ops.csa_index_topk_workspace(rows, max_csa, cfg.k), dtype=torch.uint8,
                                         device="cuda"))

    def sources(half):
        return [dict(kind="gather", kv=caches.kv_csa, off=caches.csa_off, idx=idx, n_split=sc, o_half=half),
                dict(kind="dense", kv=caches.kv_hca, off=caches.hca_off, m2=cfg.m2, w2=cfg.w2, n_split=sh,
                     o_half=half),
                dict(kind="window", kv=d["x"], off=d["tok_off"], W=cfg.W, n_split=sw, o_half=half)]

    p32 = ops.hybrid_attn(d["q"], q_pos, sources(False), cfg.scale, cfg.eps)
    p16 = ops.hybrid_attn(d["q"], q_pos, sources(True), cfg.scale, cfg.eps)
    out32 = ops.swa_merge(d["q"], None, None, None, d["sigma"], p32, 0, cfg.scale, cfg.eps, None)
    out16 = ops.swa_merge(d["q"], None, None, None, d["sigma"], p16, 0, cfg.scale, cfg.eps, None)
    # the merged call writes the same fp16 partials and merges them the same way
    outm = ops.hybrid_attn_merge(d["q"], q_pos, sources(True), d["sigma"], cfg.scale, cfg.eps)
    torch.cuda.synchronize()
    for i, ((o32, l32), (o16, l16)) in enumerate(zip(p32, p16)):
        assert o16.dtype == torch.float16 and o32.dtype == torch.float32
        assert torch.equal(l16, l32), f"source {i}: lse differs"
        a32, a16 = f64(o32), f64(o16)
        err = np.abs(a16 - a32)
        bad = err > _half_bound(a32)
        assert not bad.any(), f"source {i}: {int(bad.sum())} partial elements beyond fp16 rounding (max {err.max():.3g})"
    # merged outputs (bf16): fp16 partials move each partial element by at
    # most 2^-11 of the largest partial element, so the output (a weighted
    # mean of them, weights summing to at most 1) by at most that much before
    # its bf16 rounding, and by that plus one bf16 step after it
    ref, got = f64(out32), f64(out16)
    pmax = max(float(np.max(np.abs(f64(o)))) for o, _ in p32)
    bound = 2.0 ** -11 * pmax + 2.0 ** -7 * np.maximum(np.abs(ref), np.abs(got)) + 1e-30
    diff = np.abs(got - ref)
    assert np.all(diff <= bound), f"merged output: {int((diff > bound).sum())} elements beyond one bf16 step"
    assert torch.equal(outm, out16), "hybrid_attn_merge with fp16 partials differs from hybrid_attn + swa_merge"
    # against the oracle, every row
    idx_h = idx.cpu().numpy()
    for r in range(rows):
        g = seq_caches(caches, r)
        xs = opipe.seq_slice(raw["x"], raw["tok_off"], r)
        res = opipe.query_step(g, xs, raw["q"][r], raw["p"][r], raw["omega"][r], raw["sigma"], int(qp[r]), cfg,
                               idx=idx_h[r])
        assert_close(got[r], res["out"], cfg.dtype, f"row {r}")


def test_half_partials_rejected_on_row_tiled_path():
    """Many query rows per sequence take the row-tiled kernel, which writes
    fp32 partials only: o_half is an error there, not a silent fallback."""
    from long_context_attention_20_amd import ops
    from long_context_attention_20_amd._lib import LCAError
    cfg = li.small("half_reject", 124, (3000,), tq=24, H=128, D=512, k=512)
    raw = li.make_raw(cfg)
    d = to_device(raw, cfg)
    layer = layer_for(cfg)
    caches = layer.alloc_caches(cfg.lens, "cuda", tdtype(cfg))
    layer.compress(caches, d, d["tok_off"])
    srcs = [dict(kind="dense", kv=caches.kv_hca, off=caches.hca_off, m2=cfg.m2, w2=cfg.w2, n_split=1, o_half=True),
            dict(kind="window", kv=d["x"], off=d["tok_off"], W=cfg.W, n_split=1)]
    with pytest.raises(LCAError):
        ops.hybrid_attn(d["q"], d["q_pos"], srcs, cfg.scale, cfg.eps)
    torch.cuda.synchronize()
