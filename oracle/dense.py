"""A second, independent formulation of one query step (test infrastructure).

Pure-Python loops over every candidate key of a sequence -- every CSA entry,
every HCA entry, every raw token -- with one logit each, set to -inf where the
key is not attended (not visible, not selected, outside the window), plus the
sink, followed by a single softmax.  It shares no helper with the vectorised
oracle (its own pooling, norm, scoring, selection and softmax), so the two pin
each other on tiny inputs.  Too slow for anything but a few hundred tokens and
a handful of channels.

Same readings as the vectorised oracle (stated in its modules); rounding uses
oracle.numerics so that both see the same stored values.
"""
import math

from .numerics import round_to


def _pool(rows, zrows, C, per_channel):
    out = []
    for ch in range(C):
        zs = [zr[ch] if per_channel else zr for zr in zrows]
        zmax = max(zs)
        ws = [math.exp(z - zmax) for z in zs]
        tot = sum(ws)
        out.append(sum(wt * row[ch] for wt, row in zip(ws, rows)) / tot)
    return out


def _rms(v, eps):
    ms = sum(e * e for e in v) / len(v)
    r = 1.0 / math.sqrt(ms + eps)
    return [e * r for e in v]


def _turn(v, pos, d_rope, base):
    """Rotary embedding of one vector, pair by pair on its last d_rope dims:
    (v[a], v[a+1]) -> (v[a] cos t - v[a+1] sin t, v[a] sin t + v[a+1] cos t)
    with t = pos * base ** (-(a - lo) / d_rope), lo = len(v) - d_rope."""
    if not d_rope:
        return list(v)
    n = len(v)
    d = min(d_rope, n)
    lo = n - d
    out = list(v)
    for a in range(lo, n, 2):
        t = pos * base ** (-(a - lo) / d)
        c, s = math.cos(t), math.sin(t)
        out[a] = v[a] * c - v[a + 1] * s
        out[a + 1] = v[a] * s + v[a + 1] * c
    return out


def _entries(src, z, m, w, norm, eps, per_channel, turn=None, src2=None, z2=None):
    """With src2 (the dual-stream form): token t of window j comes from
    (src, z) when t - j*m < m, else from (src2, z2)."""
    L = len(src)
    C = len(src[0])
    out = []
    j = 0
    while j * m + w <= L:
        rows, zrows = [], []
        for t in range(j * m, j * m + w):
            second = src2 is not None and t - j * m >= m
            rows.append(src2[t] if second else src[t])
            zrows.append(z2[t] if second else z[t])
        e = _pool(rows, zrows, C, per_channel)
        e = _rms(e, eps) if norm else e
        out.append(turn(e, j * m + w - 1) if turn else e)
        j += 1
    return out


def query(x, a, g, u, c, q, p, omega, sigma, i, cfg, opt=None):
    """x,a,g: [L][D]; u,c: [L][dI]; q: [H][D]; p: [HI][dI]; omega: [HI];
    sigma: [H]; i: query position; opt: the option streams (x_b, a_b, u_b,
    c_b for the dual-stream form; v, v_b for separate values).  Returns the
    mode-A output [H][D] (float64, before the final rounding to the storage
    type) and the selected CSA entry set."""
    eps, dt = cfg.eps, cfg.dtype
    opt = opt or {}
    x = [list(map(float, r)) for r in x]
    pc = cfg.logit_per_channel
    rnd = lambda v: [float(t) for t in round_to(v, dt)]  # noqa: E731
    dr, base = getattr(cfg, "rope", 0), getattr(cfg, "rope_base", 10000.0)
    turn = (lambda v, pos: _turn(v, pos, dr, base)) if dr else None  # noqa: E731
    dual, sepv = getattr(cfg, "dual", False), getattr(cfg, "sepv", False)
    sec = (lambda k: opt[k]) if dual else (lambda k: None)  # noqa: E731
    kv_csa = [rnd(e) for e in _entries(x, a, cfg.m, cfg.w, True, eps, pc, turn, sec("x_b"), sec("a_b"))]
    ikey = [rnd(e) for e in _entries(u, c, cfg.m, cfg.w, False, eps, pc, None, sec("u_b"), sec("c_b"))]
    kv_hca = [rnd(e) for e in _entries(x, g, cfg.m2, cfg.w2, True, eps, pc, turn)]
    if sepv:
        vt = [list(map(float, r)) for r in opt["v"]]
        val_csa = [rnd(e) for e in _entries(vt, a, cfg.m, cfg.w, True, eps, pc, turn, sec("v_b"), sec("a_b"))]
        val_hca = [rnd(e) for e in _entries(vt, g, cfg.m2, cfg.w2, True, eps, pc, turn)]
    else:
        vt, val_csa, val_hca = x, kv_csa, kv_hca

    # indexer over visible entries: window end j*m + w - 1 <= i
    cand = []
    for j, key in enumerate(ikey):
        if j * cfg.m + cfg.w - 1 <= i:
            s = 0.0
            for r in range(len(p)):
                d = sum(float(p[r][t]) * key[t] for t in range(len(key)))
                s += float(omega[r]) * (d if d > 0.0 else 0.0)
            cand.append((s, j))
    cand.sort(key=lambda sj: (-sj[0], sj[1]))
    chosen = {j for _, j in cand[:cfg.k]}

    keys, vals, mask = [], [], []
    for j, e in enumerate(kv_csa):
        keys.append(e)
        vals.append(val_csa[j])
        mask.append(j in chosen)
    for j, e in enumerate(kv_hca):
        keys.append(e)
        vals.append(val_hca[j])
        mask.append(j * cfg.m2 + cfg.w2 - 1 <= i)
    for t in range(len(x)):
        xn, vn = _rms(x[t], eps), _rms(vt[t], eps)
        keys.append(rnd(turn(xn, t) if turn else xn))
        vals.append(rnd(turn(vn, t) if turn else vn))
        mask.append(i - cfg.W + 1 <= t <= i)

    out = []
    for h in range(len(q)):
        qn = _rms([float(v) for v in q[h]], eps)
        qh = rnd(turn(qn, i) if turn else qn)
        lg = []
        for key, on in zip(keys, mask):
            lg.append(cfg.scale * sum(qa * kb for qa, kb in zip(qh, key)) if on else -math.inf)
        lg.append(float(sigma[h]))
        mx = max(lg)
        ex = [math.exp(v - mx) if v != -math.inf else 0.0 for v in lg]
        den = sum(ex)
        row = [0.0] * len(keys[0])
        for e_w, val in zip(ex[:-1], vals):
            if e_w:
                for d in range(len(row)):
                    row[d] += e_w * val[d]
        row = [v / den for v in row]
        out.append(turn(row, -i) if turn else row)
    return out, chosen
