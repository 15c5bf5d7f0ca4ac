"""Pure-Python brute force for tiny inputs (test infrastructure).

An independent second implementation of the layer that shares no arithmetic
with ``oracle.moe``: plain loops over Python floats (IEEE double), subsets
enumerated exhaustively instead of sorted, and the expert-major order built by
scanning instead of by a sort.  Used on T <= 64, N <= 16 to pin the oracle.
"""
from __future__ import annotations

import itertools
import math


def dot(a, b) -> float:
    s = 0.0
    for u, v in zip(a, b):
        s += u * v
    return s


def logits(x, wg, bias=None):
    out = []
    for row in x:
        lt = [dot(row, wrow) for wrow in wg]
        if bias is not None:
            lt = [v + float(b) for v, b in zip(lt, bias)]
        out.append(lt)
    return out


def _precedes(sa, a, sb, b) -> bool:
    """Order used everywhere: larger score first, ties to the lower index."""
    return sa > sb or (sa == sb and a < b)


def _best_subset(scores, items, m):
    """The unique m-subset of ``items`` whose every member precedes every
    non-member; found by trying all subsets."""
    found = None
    for sub in itertools.combinations(items, m):
        ss = set(sub)
        rest = [i for i in items if i not in ss]
        if all(_precedes(scores[a], a, scores[b], b) for a in sub for b in rest):
            assert found is None
            found = sub
    return list(found)


def _ordered(scores, sub):
    """Members of ``sub`` ordered by counting how many members precede each."""
    ranked = [None] * len(sub)
    for a in sub:
        r = sum(1 for b in sub if b != a and _precedes(scores[b], b, scores[a], a))
        ranked[r] = a
    return ranked


def route_token(lt, N, k, n_groups=0, topk_groups=0, score_k=2, gate="sparse"):
    items = list(range(N))
    if n_groups > 1:
        gsz = N // n_groups
        gs = []
        for g in range(n_groups):
            vals = [lt[e] for e in range(g * gsz, (g + 1) * gsz)]
            best = []
            for _ in range(score_k):          # selection by repeated max scan
                mi = max(range(len(vals)), key=lambda i: (vals[i], -i))
                best.append(vals[mi])
                vals = vals[:mi] + vals[mi + 1:]
            gs.append(sum(best))
        groups = _best_subset(gs, list(range(n_groups)), topk_groups)
        items = [e for g in sorted(groups) for e in range(g * gsz, (g + 1) * gsz)]
    sel = _ordered(lt, _best_subset(lt, items, k))
    if gate == "full":                    # the selected experts' probabilities over all N
        m = max(lt)
        s = sum(math.exp(v - m) for v in lt)
        return sel, [math.exp(lt[e] - m) / s for e in sel]
    m = lt[sel[0]]
    z = [math.exp(lt[e] - m) for e in sel]
    s = sum(z)
    return sel, [v / s for v in z]


def stats(lg, idx, N, k, capacity, alpha):
    T = len(lg)
    counts = [0] * N
    for row in idx:
        for e in row:
            counts[e] += 1
    kept = [min(c, capacity) if capacity > 0 else c for c in counts]
    p = [0.0] * N
    for lt in lg:
        m = max(lt)
        z = [math.exp(v - m) for v in lt]
        s = sum(z)
        for e in range(N):
            p[e] += z[e] / s
    p = [v / T for v in p]
    f = [c / (T * k) for c in counts]
    laux = alpha * N * sum(a * b for a, b in zip(f, p))
    return counts, kept, f, p, laux


def plan(idx, N, capacity):
    """Scan experts in order; within an expert scan tokens in order."""
    T, k = len(idx), len(idx[0]) if idx else 0
    pos = [[-1] * k for _ in range(T)]
    src = []
    for e in range(N):
        taken = 0
        for t in range(T):
            for j in range(k):
                if idx[t][j] == e:
                    if capacity <= 0 or taken < capacity:
                        pos[t][j] = len(src)
                        src.append(t)
                    taken += 1
    # offsets from the kept counts
    offsets = [0]
    for e in range(N):
        n = sum(1 for t in range(T) for j in range(k) if idx[t][j] == e and pos[t][j] >= 0)
        offsets.append(offsets[-1] + n)
    return offsets, pos, src


def act(kind, u, g=None):
    if kind == "relu":
        return u if u > 0 else 0.0
    s = u / (1.0 + math.exp(-u)) if u > -700 else 0.0
    return s if kind == "silu" else s * g


def ffn(kind, a, w1, w3, w2):
    F = len(w1)
    h = []
    for f in range(F):
        u = dot(a, w1[f])
        g = dot(a, w3[f]) if w3 is not None else None
        h.append(act(kind, u, g))
    return [dot(h, w2[i]) for i in range(len(w2))]


def forward(wl, x, wg, bias, w1, w3, w2, ws=None, xq=None):
    """x etc. as nested lists of floats.  ``xq`` (optional) are the rows the
    routed experts see (the dequantised fp8 rows); ``ws`` = (ws1, ws3, ws2)."""
    lg = logits(x, wg, bias)
    idx, w = [], []
    for lt in lg:
        s, ww = route_token(lt, wl.N, wl.k, wl.n_groups, wl.topk_groups, wl.group_score_k,
                            getattr(wl, "gate", "sparse"))
        idx.append(s)
        w.append(ww)
    counts, kept, f, p, laux = stats(lg, idx, wl.N, wl.k, wl.capacity, wl.alpha)
    offsets, pos, src = plan(idx, wl.N, wl.capacity)
    xin = xq if xq is not None else x
    y = []
    for t in range(len(x)):
        acc = [0.0] * wl.d
        for j in range(wl.k):
            e = idx[t][j]
            if pos[t][j] >= 0:
                o = ffn(wl.act, xin[t], w1[e], w3[e] if w3 is not None else None, w2[e])
            elif wl.drop == "passthrough":
                o = x[t]
            elif wl.drop == "fallback":
                o = ffn(wl.act, x[t], ws[0], ws[1], ws[2])
            else:
                o = [0.0] * wl.d
            for i in range(wl.d):
                acc[i] += w[t][j] * o[i]
        if ws is not None:
            s = ffn(wl.act, x[t], ws[0], ws[1], ws[2])
            for i in range(wl.d):
                acc[i] += s[i]
        y.append(acc)
    return {"logits": lg, "idx": idx, "w": w, "counts": counts, "kept_counts": kept,
            "f": f, "p": p, "l_aux": laux, "offsets": offsets, "pos": pos, "src": src, "y": y}
