"""Pins of the CPU oracle against facts fixed outside the oracle itself:
constants and entry counts the pages and workloads state, closed forms,
library routines it must reduce to, invariants, and an independent brute-force
formulation on tiny inputs.  Each pin is chosen so that a plausible slip (a
dropped term, a sign, an index off by one, a transposed operand) fails it."""
import json
import math
import os

import numpy as np
import pytest
import torch

import lca_inputs as li
from oracle import attention as att
from oracle import compress as cmp
from oracle import dense, indexer, numerics, pipeline, quant
from oracle import indexer as idx

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "page_constants.json")) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# constants and entry counts
# --------------------------------------------------------------------------

def test_presets_match_page_constants():
    g = _gold()
    for cfg in li.CONFIGS.values():
        assert cfg.m == g["csa_stride_m"]["value"]
        assert cfg.w == g["csa_overlapping_streams"]["value"] * cfg.m
        assert cfg.m2 == cfg.w2 == g["hca_ratio"]["value"]
        assert cfg.W == g["swa_window"]["value"]
    assert li.PRO_1M_DECODE.k == g["topk_pro"]["value"]
    assert li.FLASH_DECODE.k == li.FLASH_PREFILL.k == g["topk_flash"]["value"]
    assert li.PRO_1M_DECODE.H == g["pro_query_heads"]["value"]
    assert li.PRO_1M_DECODE.D == g["pro_head_dim"]["value"]
    assert li.FLASH_DECODE.H == g["flash_query_heads"]["value"]
    assert li.PRO_1M_DECODE.lens[0] == g["context"]["value"]
    # the two-row decode is the Pro 1M decode with one drafted token beside the main one
    assert li.PRO_1M_MTP2 == li.PRO_1M_DECODE.with_(name="pro_1m_mtp2", cfg_id=li.PRO_1M_MTP2.cfg_id, tq=2)
    # the fp8-key decode draws the same inputs as the Pro 1M decode
    assert li.PRO_1M_DECODE_FP8 == li.PRO_1M_DECODE.with_(name="pro_1m_decode_fp8", ikey="fp8")
    assert li.PRO_1M_DECODE_MXFP4 == li.PRO_1M_DECODE.with_(name="pro_1m_decode_mxfp4", ikey="mxfp4")


def test_entry_counts_match_workloads():
    for case in _gold()["workload_entry_counts"]["cases"]:
        L = case["tokens"]
        assert cmp.n_entries(L, 4, 8) == case["csa"]
        assert cmp.n_entries(L, 128, 128) == case["hca"]


def test_entry_count_matches_enumeration():
    # brute force: count windows [j*m, j*m+w) that fit inside L tokens
    for L in range(0, 300):
        for m, w in ((4, 8), (128, 128), (1, 1), (2, 4), (3, 3)):
            brute = sum(1 for j in range(L + 1) if j * m + w <= L)
            assert cmp.n_entries(L, m, w) == brute


def test_visibility_boundary():
    # an entry becomes visible exactly when the query reaches its last token
    for j in range(20):
        last = j * 4 + 7
        assert cmp.n_visible(last, 4, 8) == j + 1
        assert cmp.n_visible(last - 1, 4, 8) == j
        lastH = j * 128 + 127
        assert cmp.n_visible(lastH, 128, 128) == j + 1
        assert cmp.n_visible(lastH - 1, 128, 128) == j


# --------------------------------------------------------------------------
# pooling + norm closed forms
# --------------------------------------------------------------------------

def test_constant_stream_closed_form():
    rng = np.random.default_rng(1)
    L, C = 64, 16
    x = np.ones((L, C))
    z = rng.standard_normal((L, C))
    e = cmp.compress(x, z, 4, 8, norm=False)
    assert np.all(e == 1.0) or np.max(np.abs(e - 1.0)) < 1e-15   # weights sum to one
    en = cmp.compress(x, z, 4, 8, norm=True, eps=1e-6)
    assert np.max(np.abs(en - 1.0 / math.sqrt(1.0 + 1e-6))) < 1e-15


def test_constant_logits_give_window_mean():
    rng = np.random.default_rng(2)
    L, C = 300, 8
    x = rng.standard_normal((L, C))
    z = np.full((L, C), 0.37)
    for m, w in ((4, 8), (128, 128)):
        e = cmp.compress(x, z, m, w, norm=False)
        for j in range(e.shape[0]):
            assert np.allclose(e[j], x[j * m:j * m + w].mean(axis=0), rtol=0, atol=1e-14)
        en = cmp.compress(x, z, m, w, norm=True, eps=1e-6)
        mean = np.stack([x[j * m:j * m + w].mean(axis=0) for j in range(e.shape[0])])
        ref = mean / np.sqrt((mean ** 2).mean(axis=1, keepdims=True) + 1e-6)
        assert np.allclose(en, ref, rtol=0, atol=1e-13)


def test_dominant_logit_picks_its_token_per_channel():
    # channel c puts a +60 logit on token (c mod w) of each window -> the entry
    # equals that token in that channel (per-channel softmax, right direction)
    rng = np.random.default_rng(3)
    L, C, m, w = 64, 16, 4, 8
    x = rng.standard_normal((L, C))
    z = rng.standard_normal((L, C)) * 0.1
    tol = w * math.exp(-59.0) * np.max(np.abs(x))
    for j in range(cmp.n_entries(L, m, w)):
        zz = z.copy()
        for c in range(C):
            zz[j * m + (c % w), c] = 60.0
        e = cmp.compress(x, zz, m, w, norm=False, entries=[j])[0]
        for c in range(C):
            assert abs(e[c] - x[j * m + (c % w), c]) <= tol


def test_per_token_logits_broadcast():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((40, 6))
    zt = rng.standard_normal(40)
    a = cmp.compress(x, zt, 4, 8, norm=True)
    b = cmp.compress(x, np.repeat(zt[:, None], 6, axis=1), 4, 8, norm=True)
    assert np.array_equal(a, b)


def test_overlapping_windows_share_tokens():
    # "two overlapping streams": token t (t >= 4) feeds entries t//4 - 1 and t//4
    rng = np.random.default_rng(5)
    L, C = 40, 4
    x = rng.standard_normal((L, C))
    z = rng.standard_normal((L, C))
    base = cmp.compress(x, z, 4, 8, norm=False)
    for t in range(L):
        x2 = x.copy()
        x2[t] += 1.0
        changed = np.nonzero(np.any(cmp.compress(x2, z, 4, 8, norm=False) != base, axis=1))[0]
        expect = [j for j in (t // 4 - 1, t // 4) if 0 <= j < base.shape[0]]
        assert list(changed) == expect


def test_rmsnorm_mean_square():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((50, 64)) * rng.uniform(0.01, 10, size=(50, 1))
    eps = 1e-6
    y = cmp.rmsnorm(v, eps)
    ms = (v ** 2).mean(axis=1)
    assert np.allclose((y ** 2).mean(axis=1), ms / (ms + eps), rtol=1e-13, atol=0)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(7)
    x32 = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                          np.float32([1.00390625, 1.01171875, -3.0078125, 0.0, 1e-3])])
    ours = numerics.round_bf16(x32.astype(np.float64))
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


# --------------------------------------------------------------------------
# indexer and top-k
# --------------------------------------------------------------------------

def test_indexer_single_head_is_relu_dot():
    rng = np.random.default_rng(8)
    keys = rng.standard_normal((200, 16))
    p = rng.standard_normal((1, 16))
    s = indexer.scores(p, [1.0], keys)
    brute = [max(0.0, sum(float(p[0, t]) * float(keys[j, t]) for t in range(16))) for j in range(200)]
    assert np.allclose(s, brute, rtol=0, atol=1e-12)


def test_indexer_head_weights_and_signs():
    rng = np.random.default_rng(9)
    keys = rng.standard_normal((50, 8))
    p = rng.standard_normal((3, 8))
    om = np.array([0.5, -2.0, 1.5])
    s = indexer.scores(p, om, keys)
    for j in range(50):
        ref = 0.0
        for r in range(3):
            d = float(np.dot(p[r], keys[j]))
            ref += om[r] * (d if d > 0 else 0.0)
        assert abs(s[j] - ref) < 1e-12
    # one-hot head weights isolate one head
    s1 = indexer.scores(p, [0.0, 1.0, 0.0], keys)
    assert np.allclose(s1, np.maximum(keys @ p[1], 0.0))


def test_topk_bruteforce_with_ties():
    rng = np.random.default_rng(10)
    for trial in range(50):
        n = int(rng.integers(1, 60))
        s = rng.integers(-3, 4, size=n).astype(np.float64)   # many exact ties
        k = int(rng.integers(1, 70))
        got = list(indexer.topk(s, k))
        ref = sorted(range(n), key=lambda j: (-s[j], j))[:k]
        assert got == ref


# --------------------------------------------------------------------------
# attention: reductions to textbook attention, sink, merge
# --------------------------------------------------------------------------

def _sdpa(qhat, keys, scale):
    q = torch.from_numpy(qhat)[None]       # [1, H, D] as (batch, L=H rows, D)
    k = torch.from_numpy(keys)[None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, k, scale=scale)
    return o[0].numpy()


@pytest.mark.parametrize("branch", ["csa", "hca", "swa"])
def test_window_one_reduces_to_dense_causal_attention(branch):
    """m = w = 1 (one token per entry), k >= N, no sink, one branch alone: the
    method is dense causal attention over RMS-normalised tokens."""
    rng = np.random.default_rng(11)
    L, H, D = 37, 3, 16
    x = numerics.round_bf16(rng.standard_normal((L, D)))
    z = rng.standard_normal((L, D))
    q = rng.standard_normal((H, D))
    eps, scale = 1e-6, 1.0 / math.sqrt(D)
    qhat = att.normalize_query(q, eps, "bf16")
    for i in (0, 5, L - 1):
        keys_ref = att.normalize_tokens(x[:i + 1], eps, "bf16")
        if branch == "swa":
            cfg = li.TINY.with_(W=L + 5, D=D, dtype="bf16")
            keys = pipeline.window_keys(x, i, cfg)
        else:
            ent = numerics.round_bf16(cmp.compress(x, z, 1, 1, True, eps))
            nv = cmp.n_visible(i, 1, 1)
            if branch == "csa":
                s = indexer.scores(rng.standard_normal((2, D)), [1.0, 1.0], ent[:nv])
                sel = indexer.topk(s, 10 * L)
                assert sorted(sel) == list(range(i + 1))
                keys = ent[sel]
            else:
                keys = ent[:nv]
        o, lse = att.partial(qhat, keys, scale)
        o_ref = _sdpa(qhat, keys_ref, scale)
        assert np.allclose(np.sort(keys, axis=0), np.sort(keys_ref, axis=0))
        assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
        o2, _ = att.merge([(o, lse)], None)
        assert np.allclose(o2, o_ref, rtol=0, atol=1e-12)


def test_sink_closed_forms():
    rng = np.random.default_rng(12)
    H, D = 4, 8
    key = rng.standard_normal((1, D))
    qhat = rng.standard_normal((H, D))
    scale = 0.3
    o, _, _ = att.attend(qhat, key, scale, sigma=np.full(H, -np.inf))
    assert np.allclose(o, np.repeat(key, H, axis=0), atol=1e-15)
    o, _, _ = att.attend(qhat, key, scale, sigma=np.full(H, 60.0))
    assert np.max(np.abs(o)) < 1e-20
    lg = scale * (qhat @ key[0])
    o, _, ps = att.attend(qhat, key, scale, sigma=lg)      # sink logit == key logit
    assert np.allclose(o, 0.5 * np.repeat(key, H, axis=0), atol=1e-15)
    assert np.allclose(ps, 0.5)
    # the same through partial + merge
    part = att.partial(qhat, key, scale)
    om, _ = att.merge([part], lg)
    assert np.allclose(om, 0.5 * np.repeat(key, H, axis=0), atol=1e-15)


def test_probabilities_sum_to_one():
    rng = np.random.default_rng(13)
    qhat = rng.standard_normal((5, 16))
    keys = rng.standard_normal((30, 16))
    sig = rng.standard_normal(5)
    _, prob, ps = att.attend(qhat, keys, 0.25, sig)
    assert np.allclose(prob.sum(axis=1) + ps, 1.0, atol=1e-14)
    assert np.all(prob >= 0) and np.all(ps > 0)


def test_merge_of_any_partition_equals_one_softmax():
    rng = np.random.default_rng(14)
    H, D, n = 6, 12, 40
    qhat = rng.standard_normal((H, D))
    keys = rng.standard_normal((n, D)) * 3
    sig = rng.standard_normal(H)
    ref, _, _ = att.attend(qhat, keys, 0.7, sig)
    for trial in range(20):
        lab = rng.integers(0, 4, size=n)                       # some parts may be empty
        parts = [att.partial(qhat, keys[lab == p], 0.7) for p in range(4)]
        o, _ = att.merge(parts, sig)
        assert np.allclose(o, ref, rtol=0, atol=1e-12)
    empty = att.partial(qhat, keys[:0], 0.7)
    assert np.all(empty[1] == -np.inf) and np.all(empty[0] == 0)


def test_attention_order_invariance():
    rng = np.random.default_rng(15)
    qhat = rng.standard_normal((4, 16))
    keys = rng.standard_normal((25, 16))
    o1, l1 = att.partial(qhat, keys, 0.25)
    perm = rng.permutation(25)
    o2, l2 = att.partial(qhat, keys[perm], 0.25)
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-14)


# --------------------------------------------------------------------------
# whole-step pins on tiny inputs
# --------------------------------------------------------------------------

def _tiny_cfg(dtype="bf16", **kw):
    base = dict(H=3, D=8, HI=2, dI=4, k=5, m2=16, w2=16, W=12)
    base.update(kw)
    return li.small("pin", 900, (70, 45), tq=1, dtype=dtype, **base)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gather_oracle_equals_dense_bruteforce(dtype):
    cfg = _tiny_cfg(dtype)
    raw = li.make_raw(cfg)
    caches, _ = pipeline.run(raw, cfg)
    off = raw["tok_off"]
    for b in range(cfg.B):
        L = cfg.lens[b]
        sl = lambda k: pipeline.seq_slice(raw[k], off, b)  # noqa: E731
        for i in (L - 1, L - 9, 20, 7, 0):
            r = pipeline.query_step(caches[b], sl("x"), raw["q"][b], raw["p"][b], raw["omega"][b],
                                    raw["sigma"], i, cfg)
            od, chosen = dense.query(sl("x"), sl("a"), sl("g"), sl("u"), sl("c"), raw["q"][b],
                                     raw["p"][b], raw["omega"][b], raw["sigma"], i, cfg)
            assert set(int(j) for j in r["sel"]) == chosen
            assert np.allclose(r["out_raw"] if dtype == "f32" else r["out"], np.array(od),
                               rtol=0, atol=1e-12 if dtype == "f32" else 1e-2)
            assert np.array_equal(r["out"], numerics.round_to(np.array(od), dtype)) or \
                np.max(np.abs(r["out"] - np.array(od))) <= 2.0 ** -7 * np.max(np.abs(od))


def test_causality_nan_poison():
    """Raw inputs after the query position cannot reach its output."""
    cfg = _tiny_cfg("f32")
    raw = li.make_raw(cfg)
    caches, res = pipeline.run(raw, cfg)
    off = raw["tok_off"]
    b = 0
    L = cfg.lens[b]
    for i in (L - 1, 50, 31, 16, 15, 3):
        ref = pipeline.query_step(caches[b], pipeline.seq_slice(raw["x"], off, b), raw["q"][0],
                                  raw["p"][0], raw["omega"][0], raw["sigma"], i, cfg)
        pois = {k: v.copy() for k, v in raw.items()}
        for key in ("x", "a", "g", "u", "c"):
            pois[key][int(off[b]) + i + 1:int(off[b + 1])] = np.nan
        sl = lambda k: pipeline.seq_slice(pois[k], off, b)  # noqa: E731
        pc = pipeline.build_seq_caches(sl("x"), sl("a"), sl("g"), sl("u"), sl("c"), cfg)
        got = pipeline.query_step(pc, sl("x"), raw["q"][0], raw["p"][0], raw["omega"][0],
                                  raw["sigma"], i, cfg)
        assert np.all(np.isfinite(got["out"]))
        assert np.array_equal(got["out"], ref["out"])


def test_selected_set_matters():
    """Attending over a different visible set changes the output (the checks
    that compare outputs can see a wrong selection)."""
    cfg = _tiny_cfg("f32", k=3)
    raw = li.make_raw(cfg)
    caches, res = pipeline.run(raw, cfg)
    r = res[(0, 0)]
    off = raw["tok_off"]
    nv = len(r["scores"])
    other = [j for j in range(nv) if j not in set(r["sel"].tolist())][:3]
    alt = pipeline.query_step(caches[0], pipeline.seq_slice(raw["x"], off, 0), raw["q"][0], raw["p"][0],
                              raw["omega"][0], raw["sigma"], cfg.lens[0] - 1, cfg, idx=other)
    assert np.max(np.abs(alt["out"] - r["out"])) > 1e-3


def test_empty_branches():
    """A query before the first complete window has no CSA/HCA entries; the
    window always holds the query token itself."""
    cfg = _tiny_cfg("f32")
    raw = li.make_raw(cfg)
    caches, _ = pipeline.run(raw, cfg)
    x0 = pipeline.seq_slice(raw["x"], raw["tok_off"], 0)
    r = pipeline.query_step(caches[0], x0, raw["q"][0], raw["p"][0], raw["omega"][0], raw["sigma"], 0, cfg)
    assert len(r["sel"]) == 0
    assert np.all(r["csa"][1] == -np.inf) and np.all(r["hca"][1] == -np.inf)
    assert np.all(np.isfinite(r["out"]))
    # with a single window token the output is that normalised token times its
    # softmax weight against the sink
    key = att.normalize_tokens(x0[:1], cfg.eps, cfg.dtype)[0]
    lg = cfg.scale * (r["qhat"] @ key)
    wgt = 1.0 / (1.0 + np.exp(raw["sigma"] - lg))
    assert np.allclose(r["out_raw"], wgt[:, None] * key[None, :], atol=1e-13)


def test_generator_is_seeded_and_rounded():
    a = li.make_raw(_tiny_cfg("bf16"))
    b = li.make_raw(_tiny_cfg("bf16"))
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert np.array_equal(numerics.round_bf16(a["x"].astype(np.float64)), a["x"].astype(np.float64))
    assert abs(float(np.mean(a["x"]))) < 0.05 and abs(float(np.std(a["x"])) - 1) < 0.05


# --------------------------------------------------------------------------
# fp8 (E4M3) indexer rows
# --------------------------------------------------------------------------

def _e4m3_grid():
    """Every finite E4M3 value, decoded by torch from its bit pattern."""
    import torch
    v = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    return np.unique(v[np.isfinite(v)].astype(np.float64))


def test_e4m3_grid_is_fixed_and_midpoints_go_to_even():
    g = _e4m3_grid()
    assert g.max() == 448.0 and g.min() == -448.0 and len(g) == 253   # +-0 merge
    assert np.array_equal(quant.round_e4m3(g), g)
    pos = g[g >= 0]
    mid = (pos[:-1] + pos[1:]) / 2
    r = quant.round_e4m3(mid)
    # ties to the neighbour with an even mantissa (the even multiple of the spacing)
    import torch
    even = torch.tensor(pos).to(torch.float8_e4m3fn).view(torch.uint8).numpy() % 2 == 0
    want = np.where(even[:-1], pos[:-1], pos[1:])
    assert np.array_equal(r, want)
    assert np.array_equal(quant.round_e4m3(-mid), -want)


def test_e4m3_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000),
                        [0.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -6, 447.9, 448.0, -448.0]])
    x = np.clip(x, -448, 448)
    ref = torch.tensor(x, dtype=torch.float64).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(quant.round_e4m3(x), ref)


def test_quantize_rows_invariants():
    rng = np.random.default_rng(8)
    v = rng.standard_normal((500, 64)) * np.exp(rng.uniform(-6, 6, (500, 1)))
    v[3] = 0.0
    q, s = quant.quantize_rows(v)
    assert np.all(q[3] == 0) and s[3] == 0
    live = s > 0
    assert np.all(np.max(np.abs(q[live]), axis=1) == 448.0)          # the largest channel hits the top value
    assert np.array_equal(s, s.astype(np.float32).astype(np.float64))  # fp32 scales
    err = np.abs(quant.dequantize_rows(q, s) - v)
    # half a spacing of the E4M3 value (relative 2**-4), or half the subnormal spacing
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)


def test_fp8_scores_reduce_to_plain_scores_on_the_grid():
    """Rows already on the E4M3 grid with a power-of-two scale (and the
    largest at 448 times it) quantize exactly: the fp8 score equals the plain
    one, negative head weights included; rows off the grid score as the rows
    they stand for."""
    rng = np.random.default_rng(9)
    g = _e4m3_grid()
    keys = rng.choice(g, (300, 64)) * 2.0 ** -5
    keys[:, 0] = 448.0 * 2.0 ** -5
    p = rng.choice(g, (4, 64)) * 2.0 ** -3
    p[:, 5] = -448.0 * 2.0 ** -3
    om = np.array([1.5, -0.7, 0.25, 2.0])
    q, s = quant.quantize_rows(keys)
    assert np.all(s == 2.0 ** -5) and np.array_equal(q * s[:, None], keys)
    assert np.array_equal(quant.scores_fp8(p, om, q, s), idx.scores(p, om, keys))
    off = keys + rng.standard_normal(keys.shape) * 0.01
    q2, s2 = quant.quantize_rows(off)
    assert not np.array_equal(quant.scores_fp8(p, om, q2, s2), idx.scores(p, om, off))
    assert np.allclose(quant.scores_fp8(p, om, q2, s2), idx.scores(p, om, q2 * s2[:, None]), rtol=0, atol=0)


# --------------------------------------------------------------------------
# MXFP4 (E2M1 elements, E8M0 block scales) indexer rows
# --------------------------------------------------------------------------

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e2m1_brute(x):
    """Nearest grid value by enumeration; a tie goes to the value whose
    mantissa bit is 0 (0, 1, 2, 4)."""
    out = np.empty_like(x)
    even = {0.0: True, 0.5: False, 1.0: True, 1.5: False, 2.0: True, 3.0: False, 4.0: True, 6.0: False}
    for i, v in enumerate(np.abs(x)):
        d = np.abs(E2M1_GRID - v)
        best = np.nonzero(d == d.min())[0]
        pick = [g for g in E2M1_GRID[best] if even[g]] if len(best) > 1 else list(E2M1_GRID[best])
        out[i] = np.copysign(pick[0], x[i])
    return out


def test_e2m1_rounding_matches_brute_force():
    rng = np.random.default_rng(10)
    mids = (E2M1_GRID[:-1] + E2M1_GRID[1:]) / 2
    x = np.concatenate([rng.uniform(-6, 6, 5000), E2M1_GRID, -E2M1_GRID, mids, -mids])
    assert np.array_equal(quant.round_e2m1(x), _e2m1_brute(x))
    assert np.array_equal(quant.round_e2m1(E2M1_GRID), E2M1_GRID)


def test_mx_quantize_invariants():
    rng = np.random.default_rng(11)
    v = rng.standard_normal((300, 64)) * np.exp(rng.uniform(-5, 5, (300, 1)))
    v[5, :32] = 0.0
    q, s = quant.quantize_mx_rows(v)
    assert s.shape == (300, 2) and s[5, 0] == 2.0 ** -127 and np.all(q[5, :32] == 0)
    # power-of-two scales; the block maximum sits in [4, 8) before the clamp at 6
    live = np.ones_like(s, dtype=bool)
    live[5, 0] = False
    assert np.all(np.log2(s) == np.round(np.log2(s)))
    amax = np.max(np.abs(v.reshape(300, 2, 32)), axis=-1)
    r = amax[live] / s[live]
    assert np.all((r >= 4) & (r < 8))
    assert set(np.unique(np.abs(q))).issubset(set(E2M1_GRID.tolist()))
    # error: half a spacing of the element (at most 1 at the top binade), or the clamp from [6, 8)
    err = np.abs(quant.dequantize_mx_rows(q, s) - v).reshape(300, 2, 32) / s[..., None]
    a = np.abs(v.reshape(300, 2, 32)) / s[..., None]
    assert np.all(err <= np.where(a >= 6, a - 6, np.maximum(0.25, np.where(a >= 4, 1.0, np.where(a >= 2, 0.5, 0.25)))) + 1e-12)


def test_mx_scores_reduce_to_plain_scores_on_the_grid():
    rng = np.random.default_rng(12)
    keys = rng.choice(E2M1_GRID, (200, 64)) * rng.choice([-1, 1], (200, 64)) * 2.0 ** -3
    keys[:, 0] = 4.0 * 2.0 ** -3
    keys[:, 32] = -6.0 * 2.0 ** -3          # block maxima 4 and 6 times 2**-3: scale 2**-3
    q, s = quant.quantize_mx_rows(keys)
    assert np.all(s == 2.0 ** -3) and np.array_equal(quant.dequantize_mx_rows(q, s), keys)
    p = rng.standard_normal((4, 64))
    om = np.array([0.5, -1.0, 2.0, 0.25])
    assert np.array_equal(idx.scores(p, om, quant.dequantize_mx_rows(q, s)), idx.scores(p, om, keys))


# --------------------------------------------------------------------------
# partial rotary embedding ("DeepSeek-V4", Core block and Provenance 16)
# --------------------------------------------------------------------------

from oracle import rope  # noqa: E402


def test_rope_identity_lengths_and_untouched_dims():
    rng = np.random.default_rng(30)
    x = rng.standard_normal((5, 128))
    assert np.array_equal(rope.rotate(x, 0, 64), x)          # position 0 turns by exp(0) = 1
    y = rope.rotate(x, 12345, 64)
    assert np.array_equal(y[:, :64], x[:, :64])                # the first D - 64 dims stay
    pair = lambda v: v[:, 64::2] ** 2 + v[:, 65::2] ** 2     # noqa: E731
    assert np.allclose(pair(y), pair(x), rtol=1e-13, atol=0)  # every pair keeps its length
    # D <= 64: every dim rotates
    z = rope.rotate(x[:, :64], 9, 64)
    assert not np.allclose(z[:, :2], x[:, :2])


def test_rope_closed_form_on_basis_vectors():
    # the first rotated pair turns by pos radians (theta_0 = base**0 = 1), the
    # last by pos * base**(-62/64); (1, 0) -> (cos t, sin t), (0, 1) -> (-sin t, cos t)
    for pos in (1, 7, 1048575):
        for a, t in ((64, float(pos)), (126, pos * 10000.0 ** (-62.0 / 64.0))):
            e = np.zeros(128)
            e[a] = 1.0
            y = rope.rotate(e, pos, 64)
            assert abs(y[a] - math.cos(t)) < 1e-9 and abs(y[a + 1] - math.sin(t)) < 1e-9
            e = np.zeros(128)
            e[a + 1] = 1.0
            y = rope.rotate(e, pos, 64)
            assert abs(y[a] + math.sin(t)) < 1e-9 and abs(y[a + 1] - math.cos(t)) < 1e-9
            assert np.count_nonzero(y) == 2


def test_rope_composes_and_inverts():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((4, 96))
    for a, b in ((3, 5), (1000, -1000), (262143, 786432)):
        assert np.allclose(rope.rotate(rope.rotate(x, a, 64), b, 64), rope.rotate(x, a + b, 64), atol=1e-9)
    assert np.allclose(rope.rotate(rope.rotate(x, 777, 64), -777, 64), x, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(32)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for d in (0, 3, 127, 5000):
        vals = [rope.rotate(q, i, 64) @ rope.rotate(k, i - d, 64) for i in (d, d + 1, d + 977, 1048575)]
        assert np.allclose(vals, vals[0], rtol=0, atol=1e-9)
    assert abs(rope.rotate(q, 10, 64) @ rope.rotate(k, 0, 64) - rope.rotate(q, 11, 64) @ rope.rotate(k, 0, 64)) > 1e-6


def test_rope_single_key_output_turns_back_to_the_key():
    # one attended entry, no sink: the output is the stored (rotated) entry, and
    # the -i turn of the output gives back the unrotated key when the entry
    # sits at the query's position, or the key turned by their distance
    rng = np.random.default_rng(33)
    D, H = 64, 3
    key = cmp.rmsnorm(rng.standard_normal(D), 1e-6)
    cfg = li.TINY.with_(D=D, H=H, rope=64)
    qhat = rng.standard_normal((H, D))
    for i, j in ((500, 500), (500, 380)):
        stored = rope.rotate(key, j, 64)
        o, _, _ = att.attend(qhat, stored[None], cfg.scale, sigma=np.full(H, -np.inf))
        got = pipeline.finish(o, i, cfg)
        want = rope.rotate(key, j - i, 64)
        assert np.allclose(got, np.repeat(want[None], H, axis=0), atol=1e-6)
    assert np.allclose(pipeline.finish(np.repeat(rope.rotate(key, 500, 64)[None], H, 0), 500, cfg), key, atol=1e-6)


def test_rope_window_one_reduces_to_rotary_causal_attention():
    """m = w = 1 (one token per entry), k >= N, no sink, the CSA branch alone
    with rope: textbook rotary causal attention, the query turned by i, token j
    (key and value) by j, the output turned back by -i (torch SDPA)."""
    rng = np.random.default_rng(34)
    L, H, D = 29, 3, 16
    x = numerics.round_bf16(rng.standard_normal((L, D)))
    z = rng.standard_normal((L, D))
    q = rng.standard_normal((H, D))
    eps = 1e-6
    cfg = li.TINY.with_(D=D, H=H, dtype="f32", rope=8, m=1, w=1)
    ent = pipeline.kv_entries(x, z, 1, 1, cfg)                  # rotated by their positions j
    for i in (0, 6, L - 1):
        qhat = att.normalize_query(q, eps, "f32", pos=i, rope=8)
        o, _ = att.partial(qhat, ent[:i + 1], cfg.scale)
        got = pipeline.finish(o, i, cfg)
        # textbook: pooling with w = 1 is the token itself
        kr = np.stack([rope.rotate(cmp.rmsnorm(x[j], eps), j, 8) for j in range(i + 1)])
        qr = rope.rotate(cmp.rmsnorm(q, eps), i, 8)
        o_ref = rope.rotate(_sdpa(qr, kr, cfg.scale), -i, 8)
        assert np.allclose(got, numerics.round_f32(o_ref), rtol=0, atol=2e-6)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gather_oracle_equals_dense_bruteforce_with_rope(dtype):
    cfg = _tiny_cfg(dtype, rope=4)
    raw = li.make_raw(cfg)
    caches, _ = pipeline.run(raw, cfg)
    off = raw["tok_off"]
    for b in range(cfg.B):
        L = cfg.lens[b]
        sl = lambda k: pipeline.seq_slice(raw[k], off, b)  # noqa: E731
        for i in (L - 1, L - 9, 20, 7, 0):
            r = pipeline.query_step(caches[b], sl("x"), raw["q"][b], raw["p"][b], raw["omega"][b],
                                    raw["sigma"], i, cfg)
            od, chosen = dense.query(sl("x"), sl("a"), sl("g"), sl("u"), sl("c"), raw["q"][b],
                                     raw["p"][b], raw["omega"][b], raw["sigma"], i, cfg)
            assert set(int(j) for j in r["sel"]) == chosen
            turned = rope.rotate(r["out_raw"], -i, cfg.rope)
            assert np.allclose(turned, np.array(od), rtol=0, atol=1e-12 if dtype == "f32" else 1e-2)
            # rotation changes the output (the pins can see a missing turn)
            plain = pipeline.query_step(pipeline.build_seq_caches(sl("x"), sl("a"), sl("g"), sl("u"), sl("c"),
                                                                  cfg.with_(rope=0)),
                                        sl("x"), raw["q"][b], raw["p"][b], raw["omega"][b], raw["sigma"], i,
                                        cfg.with_(rope=0))
            if i > 0:
                assert np.max(np.abs(plain["out"] - r["out"])) > 1e-3


# --------------------------------------------------------------------------
# dual-stream compressor and separate values
# --------------------------------------------------------------------------

def _streams(seed, L=41, C=6, per_channel=True):
    rng = np.random.default_rng(seed)
    zs = (L, C) if per_channel else (L,)
    return (rng.standard_normal((L, C)), rng.standard_normal(zs), rng.standard_normal((L, C)),
            rng.standard_normal(zs))


@pytest.mark.parametrize("per_channel", [True, False])
@pytest.mark.parametrize("norm", [False, True])
def test_dual_with_equal_streams_is_the_single_stream(per_channel, norm):
    x, z, _, _ = _streams(40, per_channel=per_channel)
    single = cmp.compress(x, z, 4, 8, norm)
    dual = cmp.compress(x, z, 4, 8, norm, src2=x.copy(), z2=z.copy())
    assert dual.shape == single.shape == (cmp.n_entries(41, 4, 8), 6)
    assert np.array_equal(dual, single)


@pytest.mark.parametrize("per_channel", [True, False])
def test_dual_halves_come_from_their_streams(per_channel):
    """With one half's logits pushed to -1e4 (weights underflow to zero) an
    entry is the pool of the other half alone: entry j of the non-overlapping
    pool (w = m) of the first stream, or entry j + 1 of that of the second."""
    x, z, x2, z2 = _streams(41, per_channel=per_channel)
    n = cmp.n_entries(41, 4, 8)
    first_only = cmp.compress(x, z, 4, 8, False, src2=x2, z2=z2 - 1e4)
    assert np.allclose(first_only, cmp.compress(x, z, 4, 4, False)[:n], rtol=0, atol=1e-15)
    second_only = cmp.compress(x, z - 1e4, 4, 8, False, src2=x2, z2=z2)
    assert np.allclose(second_only, cmp.compress(x2, z2, 4, 4, False)[1:n + 1], rtol=0, atol=1e-15)
    # the two halves really differ (a swapped half fails one of the above)
    assert np.max(np.abs(first_only - second_only)) > 0.1


def test_dual_closed_form_on_constant_streams():
    """Constant first-half rows c1 with logit 0 and second-half rows c2 with
    logit log 3: every entry is (c1 + 3 c2) / 4 per channel."""
    L, C = 30, 5
    c1, c2 = np.arange(1.0, C + 1), -2.0 * np.arange(1.0, C + 1)
    x, x2 = np.tile(c1, (L, 1)), np.tile(c2, (L, 1))
    z, z2 = np.zeros((L, C)), np.full((L, C), math.log(3.0))
    e = cmp.compress(x, z, 4, 8, False, src2=x2, z2=z2)
    assert np.allclose(e, np.tile((c1 + 3 * c2) / 4, (cmp.n_entries(L, 4, 8), 1)), rtol=0, atol=1e-14)
    with pytest.raises(ValueError):
        cmp.compress(x, z, 4, 4, False, src2=x2, z2=z2)   # no overlap: no second half


def _sdpa_v(qhat, keys, vals, scale):
    q = torch.from_numpy(np.ascontiguousarray(qhat))[None]
    k = torch.from_numpy(np.ascontiguousarray(keys))[None]
    v = torch.from_numpy(np.ascontiguousarray(vals))[None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[0].numpy()


def test_separate_values_partial_is_textbook_attention():
    rng = np.random.default_rng(42)
    H, D, n = 5, 12, 23
    qhat, keys, vals = rng.standard_normal((H, D)), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    o, lse = att.partial(qhat, keys, 0.4, vals)
    assert np.allclose(o, _sdpa_v(qhat, keys, vals, 0.4), rtol=0, atol=1e-12)
    # the weights are the keys' (lse does not depend on the values)
    assert np.array_equal(lse, att.partial(qhat, keys, 0.4)[1])
    # constant values come out unchanged; with a sink they are scaled by the
    # probability mass of the keys
    c = rng.standard_normal(D)
    oc, _ = att.partial(qhat, keys, 0.4, np.tile(c, (n, 1)))
    assert np.allclose(oc, np.tile(c, (H, 1)), rtol=0, atol=1e-13)
    sig = rng.standard_normal(H)
    o_s, prob, ps = att.attend(qhat, keys, 0.4, sig, values=np.tile(c, (n, 1)))
    assert np.allclose(o_s, (1.0 - ps)[:, None] * c[None], rtol=0, atol=1e-13)
    with pytest.raises(ValueError):
        att.partial(qhat, keys, 0.4, vals[:-1])


def test_separate_values_window_one_reduces_to_causal_attention():
    """m = w = 1, k >= N, one branch: textbook causal attention with keys the
    normalised x tokens and values the normalised v tokens (torch SDPA)."""
    rng = np.random.default_rng(43)
    L, H, D = 31, 3, 16
    x = numerics.round_bf16(rng.standard_normal((L, D)))
    v = numerics.round_bf16(rng.standard_normal((L, D)))
    z, g = rng.standard_normal((L, D)), rng.standard_normal((L, D))
    u, c = rng.standard_normal((L, 4)), rng.standard_normal((L, 4))
    q = rng.standard_normal((H, D))
    cfg = li.TINY.with_(D=D, H=H, dI=4, dtype="f32", m=1, w=1, m2=1, w2=1, k=4 * L, W=L + 3, sepv=True)
    caches = pipeline.build_seq_caches(x, z, g, u, c, cfg, {"v": v})
    for i in (0, 7, L - 1):
        r = pipeline.query_step(caches, x, q, rng.standard_normal((2, 4)), np.ones(2), np.full(H, -np.inf), i, cfg,
                                v_seq=v)
        qhat = att.normalize_query(q, cfg.eps, "f32")
        kref = np.stack([cmp.rmsnorm(x[j], cfg.eps) for j in range(i + 1)])
        vref = np.stack([cmp.rmsnorm(v[j], cfg.eps) for j in range(i + 1)])
        o_ref = _sdpa_v(qhat, kref, vref, cfg.scale)
        for branch in ("csa", "hca", "swa"):
            assert np.allclose(r[branch][0], o_ref, rtol=0, atol=1e-6), branch
        # the keys' own average differs (the values are really used)
        assert i == 0 or np.max(np.abs(_sdpa_v(qhat, kref, kref, cfg.scale) - o_ref)) > 1e-2


@pytest.mark.parametrize("dtype,d_rope", [("bf16", 0), ("f32", 0), ("f32", 4)])
@pytest.mark.parametrize("dual,sepv", [(True, False), (False, True), (True, True)])
def test_options_oracle_equals_dense_bruteforce(dtype, d_rope, dual, sepv):
    cfg = _tiny_cfg(dtype, rope=d_rope, dual=dual, sepv=sepv)
    raw = li.make_raw(cfg)
    caches, _ = pipeline.run(raw, cfg)
    off = raw["tok_off"]
    for b in range(cfg.B):
        L = cfg.lens[b]
        sl = lambda k: pipeline.seq_slice(raw[k], off, b)  # noqa: E731
        opt = {k: sl(k) for k in pipeline.OPTION_STREAMS if k in raw}
        for i in (L - 1, L - 9, 20, 7, 0):
            r = pipeline.query_step(caches[b], sl("x"), raw["q"][b], raw["p"][b], raw["omega"][b],
                                    raw["sigma"], i, cfg, v_seq=opt.get("v"))
            od, chosen = dense.query(sl("x"), sl("a"), sl("g"), sl("u"), sl("c"), raw["q"][b],
                                     raw["p"][b], raw["omega"][b], raw["sigma"], i, cfg, opt)
            assert set(int(j) for j in r["sel"]) == chosen
            got = rope.rotate(r["out_raw"], -i, cfg.rope) if cfg.rope else r["out_raw"]
            assert np.allclose(got, np.array(od), rtol=0, atol=1e-12 if dtype == "f32" else 1e-2)
    # the option changes the result (the pins can see it ignored)
    plain, _ = pipeline.run(raw, cfg.with_(dual=False, sepv=False))
    assert any(np.max(np.abs(plain[b].kv_csa - caches[b].kv_csa)) > 1e-3 for b in range(cfg.B)) or not dual
    assert all(caches[b].v_csa is not None for b in range(cfg.B)) or not sepv
