"""Pure-Python brute force of the MoE layer, for tiny shapes only.

Independent of ``oracle.moe``: plain loops over Python floats with
``math.exp``, no numpy arithmetic, selection by repeated scans instead of a
sort.  It follows the same plain reading of the pages as ``oracle.moe`` (see
the package docstring) so the two can be compared value by value.
"""
from __future__ import annotations

import math


def _dot(a, b):
    s = 0.0
    for u, v in zip(a, b):
        s += u * v
    return s


def route_one(x, Wr, b, k):
    """One token: logits, softmax, top-k by repeated maximum scans, renormalisation."""
    E = len(Wr)
    l = [_dot(x, Wr[e]) + (0.0 if b is None else float(b[e])) for e in range(E)]
    m = max(l)
    z = [math.exp(v - m) for v in l]
    zs = sum(z)
    p = [v / zs for v in z]
    chosen = []
    for _ in range(k):
        best = None
        for e in range(E):
            if e in chosen:
                continue
            if best is None or l[e] > l[best]:   # strict: equal logits keep the lower index
                best = e
        chosen.append(best)
    ps = sum(p[e] for e in chosen)
    w = [p[e] / ps for e in chosen]
    return l, p, chosen, w


def ffn_one(x, Wg, Wu, Wd):
    """One token through one SwiGLU expert: Wd (silu(Wg x) * (Wu x))."""
    a = []
    for i in range(len(Wg)):
        g = _dot(x, Wg[i])
        u = _dot(x, Wu[i])
        a.append(g / (1.0 + math.exp(-g)) * u)
    return [_dot(a, Wd[h]) for h in range(len(Wd))]


def moe_forward(x, Wr, b, Wg, Wu, Wd, k, shared=None):
    """All tokens: returns (out, ids, w) as nested Python lists."""
    out, all_ids, all_w = [], [], []
    for xt in x:
        _, _, ids, w = route_one(xt, Wr, b, k)
        acc = [0.0] * len(xt)
        for e, we in zip(ids, w):
            y = ffn_one(xt, Wg[e], Wu[e], Wd[e])
            acc = [a + we * v for a, v in zip(acc, y)]
        if shared is not None:
            Wsg, Wsu, Wsd = shared
            for s in range(len(Wsg)):
                y = ffn_one(xt, Wsg[s], Wsu[s], Wsd[s])
                acc = [a + v for a, v in zip(acc, y)]
        out.append(acc)
        all_ids.append(ids)
        all_w.append(w)
    return out, all_ids, all_w


def dispatch(ids, E, M):
    """Expert-sorted order by brute force: for each expert, scan all flat ids in order."""
    T, k = len(ids), len(ids[0])
    n = T * k
    flat = [ids[t][j] for t in range(T) for j in range(k)]
    counts = [sum(1 for e2 in flat if e2 == e) for e in range(E)]
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + -(-counts[e] // M) * M)
    cap = -(-(n + E * (M - 1)) // M) * M
    sorted_ids = [n] * cap
    inv = [None] * n
    for e in range(E):
        r = 0
        for f in range(n):
            if flat[f] == e:
                sorted_ids[offsets[e] + r] = f
                inv[f] = offsets[e] + r
                r += 1
    tile_expert = []
    for i in range(cap // M):
        owner = -1
        for e in range(E):
            if offsets[e] <= i * M < offsets[e + 1]:
                owner = e
        tile_expert.append(owner)
    active = [e for e in range(E) if counts[e] > 0]
    return dict(counts=counts, offsets=offsets, sorted_ids=sorted_ids,
                tile_expert=tile_expert, inv=inv, active=active, capacity=cap)


def sparse_ffn_one(x, Wg, Wu, Wd, scores, c):
    """Brute force: rank channels by score (higher first, equal scores by
    lower index, NaN below every number), keep the first c, and sum their
    contributions one by one."""
    I = len(Wg)

    def rank_key(i):
        v = scores[i]
        return (1, 0.0, i) if math.isnan(v) else (0, -v, i)

    ranked = sorted(range(I), key=rank_key)[:c]
    y = [0.0] * len(x)
    for i in ranked:
        g = _dot(Wg[i], x)
        u = _dot(Wu[i], x)
        a = g / (1.0 + math.exp(-g)) * u
        for h in range(len(x)):
            y[h] += Wd[h][i] * a
    return y
