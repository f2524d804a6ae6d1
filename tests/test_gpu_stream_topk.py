"""The streaming selection of many query rows (csa_index_topk with no scores
requested: scores and exact top-k in one launch, no score stored) against
the two-launch path that stores every score (csa_index_score then
csa_topk_select), and against the oracle on sampled rows.

Both paths compute bit-identical fp32 scores (the same row-tiled products),
so their selections must be identical lists; against the oracle, the
selection is the exact top-k of the GPU's own scores and differs from the
oracle's only at near ties (the rule of check_topk)."""
import numpy as np
import pytest
import torch

import lca_inputs as li
from oracle import compress as ocmp
from oracle import indexer as oidx
from gpu_util import check_topk, key_rows, layer_for, score_bound, tdtype, to_device

pytestmark = pytest.mark.gpu

# name: (lens, tq, HI, dI, k, key format, planted runs)
CASES = {
    # three sequences, row groups of 16 + 16 + 8, a sequence with fewer
    # entries than k (every row takes all it sees)
    "ragged_b3": ((9000, 4101, 777), 40, 4, 64, 256, "bf16", 0),
    # lists shrunk many times (about 5000 entries, 128 kept)
    "shrink_hi2": ((20000,), 48, 2, 128, 128, "bf16", 0),
    # few keys kept per list: the final passes see lists shorter than a wave
    "k1_hi1": ((6000,), 32, 1, 32, 1, "bf16", 0),
    "k8": ((6000,), 32, 4, 64, 8, "bf16", 0),
    "k512": ((40000,), 33, 4, 64, 512, "bf16", 0),
    # k above the streaming selection's bound: the call stores the scores
    # in its workspace and selects in a launch of its own (same lists)
    "k1024": ((40000,), 33, 4, 64, 1024, "bf16", 0),
    # identical planted keys: exact score ties inside every row
    "planted": ((30000,), 32, 4, 64, 512, "bf16", 32),
    "fp8": ((9000, 4101), 40, 4, 64, 256, "fp8", 0),
    "mxfp4": ((9000, 4101), 40, 4, 64, 256, "mxfp4", 0),
}


def _setup(name):
    lens, tq, HI, dI, k, fmt, plant = CASES[name]
    cfg = li.small(f"stream_{name}", 140, lens, tq=tq, H=16, D=64, HI=HI, dI=dI, k=k, ikey=fmt, plant=plant, W=16)
    raw = li.make_raw(cfg)
    d = to_device(raw, cfg)
    layer = layer_for(cfg)
    caches = layer.alloc_caches(cfg.lens, "cuda", tdtype(cfg))
    layer.compress(caches, d, d["tok_off"], which=("idx",))
    torch.cuda.synchronize()
    return cfg, raw, d, layer, caches


def _both(cfg, d, layer, caches, ikey=None):
    from long_context_attention_20_amd import ops
    ikey = caches.ikey if ikey is None else ikey
    maxN = ocmp.n_entries(max(cfg.lens), cfg.m, cfg.w)
    rows = cfg.B * cfg.tq
    ws = layer.index_workspace(rows, maxN, "cuda")
    idx_s = ops.csa_index_topk(d["p"], d["omega"], ikey, caches.csa_off, d["q_pos"], cfg.k, cfg.m, cfg.w, maxN, ws)
    sc = torch.full((rows, maxN), float("nan"), dtype=torch.float32, device="cuda")
    ws2 = layer.index_workspace(rows, maxN, "cuda").clone()
    idx_t = ops.csa_index_topk(d["p"], d["omega"], ikey, caches.csa_off, d["q_pos"], cfg.k, cfg.m, cfg.w, maxN, ws2,
                               scores=sc)
    torch.cuda.synchronize()
    return idx_s.cpu().numpy(), idx_t.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_stream_topk_equals_stored_scores_path(name):
    cfg, raw, d, layer, caches = _setup(name)
    print(f"[stream top-k] {name}: lens={cfg.lens} tq={cfg.tq} HI={cfg.HI} dI={cfg.dI} k={cfg.k} keys={cfg.ikey}",
          flush=True)
    idx_s, idx_t, sc = _both(cfg, d, layer, caches)
    assert np.array_equal(idx_s, idx_t), f"{name}: streaming selection differs from the stored-scores path"
    # against the oracle: every 5th row, the first and the last row of each sequence
    keys = key_rows(caches.ikey, cfg.dI)
    co = caches.csa_off_h
    for b in range(cfg.B):
        for t in sorted(set(range(0, cfg.tq, 5)) | {cfg.tq - 1}):
            r = b * cfg.tq + t
            nv = ocmp.n_visible(int(raw["q_pos"][b, t]), cfg.m, cfg.w)
            sel = idx_s[r][idx_s[r] >= 0]
            assert len(sel) == min(cfg.k, nv) and np.all(np.diff(sel) > 0), f"row {r}: not ascending"
            kb = keys[co[b]:co[b] + nv]
            p64 = raw["p"][r].astype(np.float64)
            om = raw["omega"][r].astype(np.float64)
            check_topk(idx_s[r], sc[r], oidx.scores(p64, om, kb), score_bound(p64, om, kb), cfg.k)


def test_stream_topk_all_scores_equal():
    """Every key identical: all of a row's scores are equal, the selection is
    its k smallest entries (ties go to the smaller index) -- the shrinking
    and the final selection then decide on the entry part of the keys alone."""
    cfg, raw, d, layer, caches = _setup("shrink_hi2")
    ikey = caches.ikey.clone()
    ikey[:] = ikey[7]
    idx_s, idx_t, _ = _both(cfg, d, layer, caches, ikey)
    assert np.array_equal(idx_s, idx_t)
    for r in range(cfg.B * cfg.tq):
        nv = ocmp.n_visible(int(raw["q_pos"].reshape(-1)[r]), cfg.m, cfg.w)
        want = np.arange(min(cfg.k, nv))
        assert np.array_equal(idx_s[r][:len(want)], want), f"row {r}: not the first k entries"
