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


def _entries(src, z, m, w, norm, eps, per_channel):
    L = len(src)
    C = len(src[0])
    out = []
    j = 0
    while j * m + w <= L:
        e = _pool(src[j * m:j * m + w], z[j * m:j * m + w], C, per_channel)
        out.append(_rms(e, eps) if norm else e)
        j += 1
    return out


def query(x, a, g, u, c, q, p, omega, sigma, i, cfg):
    """x,a,g: [L][D]; u,c: [L][dI]; q: [H][D]; p: [HI][dI]; omega: [HI];
    sigma: [H]; i: query position.  Returns the mode-A output [H][D] (float64,
    before the final rounding to the storage type) and the selected CSA entry
    set."""
    eps, dt = cfg.eps, cfg.dtype
    x = [list(map(float, r)) for r in x]
    pc = cfg.logit_per_channel
    rnd = lambda v: [float(t) for t in round_to(v, dt)]  # noqa: E731
    kv_csa = [rnd(e) for e in _entries(x, a, cfg.m, cfg.w, True, eps, pc)]
    ikey = [rnd(e) for e in _entries(u, c, cfg.m, cfg.w, False, eps, pc)]
    kv_hca = [rnd(e) for e in _entries(x, g, cfg.m2, cfg.w2, True, eps, pc)]

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

    keys, mask = [], []
    for j, e in enumerate(kv_csa):
        keys.append(e)
        mask.append(j in chosen)
    for j, e in enumerate(kv_hca):
        keys.append(e)
        mask.append(j * cfg.m2 + cfg.w2 - 1 <= i)
    for t in range(len(x)):
        keys.append(rnd(_rms(x[t], eps)))
        mask.append(i - cfg.W + 1 <= t <= i)

    out = []
    for h in range(len(q)):
        qh = rnd(_rms([float(v) for v in q[h]], eps))
        lg = []
        for key, on in zip(keys, mask):
            lg.append(cfg.scale * sum(qa * kb for qa, kb in zip(qh, key)) if on else -math.inf)
        lg.append(float(sigma[h]))
        mx = max(lg)
        ex = [math.exp(v - mx) if v != -math.inf else 0.0 for v in lg]
        den = sum(ex)
        row = [0.0] * len(keys[0])
        for e_w, key in zip(ex[:-1], keys):
            if e_w:
                for d in range(len(row)):
                    row[d] += e_w * key[d]
        out.append([v / den for v in row])
    return out, chosen
