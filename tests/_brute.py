"""Pure-Python brute force for tiny inputs (lists of floats, math.exp).

Written independently of the oracle: top-k by enumerating every subset,
gates by the softmax-over-all-then-renormalise route, FFNs by explicit loops.
Used only to pin the oracle on tiny shapes.
"""

import itertools
import math
import struct


def f32(v):
    """Round a Python float to the nearest binary32 (the decision precision)."""
    return struct.unpack("f", struct.pack("f", v))[0]


def matvec_rows(x, w_router):
    """logits[t][e] = sum_j x[t][j] * w[j][e] with exact-ish fsum."""
    T, d, N = len(x), len(x[0]), len(w_router[0])
    return [[math.fsum(x[t][j] * w_router[j][e] for j in range(d)) for e in range(N)]
            for t in range(T)]


def sig(z):
    return 1.0 / (1.0 + math.exp(-z)) if z >= 0 else math.exp(z) / (1.0 + math.exp(z))


def best_subset(scores, k):
    """Enumerate all k-subsets; keep those whose every member scores >= every
    non-member (float32 scores); among those, prefer lower indices on ties.
    Returns the subset ordered best first (score desc, index asc)."""
    N = len(scores)
    s = [f32(v) for v in scores]
    valid = []
    for sub in itertools.combinations(range(N), k):
        rest = [e for e in range(N) if e not in sub]
        if not rest or min(s[e] for e in sub) >= max(s[e] for e in rest):
            valid.append(sorted(sub, key=lambda e: (-s[e], e)))
    # lower indices win ties: compare the (score desc, index asc) keys
    valid.sort(key=lambda sub: [(-s[e], e) for e in sub])
    return valid[0]


def route_softmax_all_renorm(logits_row, k):
    """Softmax over all N, keep top-k, renormalise the survivors."""
    m = max(logits_row)
    p = [math.exp(v - m) for v in logits_row]
    tot = math.fsum(p)
    p = [v / tot for v in p]
    sel = best_subset(logits_row, k)
    keep = math.fsum(p[e] for e in sel)
    return sel, [p[e] / keep for e in sel]


def route_sigmoid_bias(logits_row, k, bias):
    a = [sig(v) for v in logits_row]
    u = [a[e] + bias[e] for e in range(len(a))]
    sel = best_subset(u, k)
    tot = math.fsum(a[e] for e in sel)
    return sel, [a[e] / tot for e in sel]


def swiglu(xrow, wg, wu, wd):
    d_ff, d = len(wg), len(xrow)
    h = []
    for n in range(d_ff):
        g = math.fsum(wg[n][j] * xrow[j] for j in range(d))
        u = math.fsum(wu[n][j] * xrow[j] for j in range(d))
        h.append(g * sig(g) * u)
    return [math.fsum(wd[o][n] * h[n] for n in range(d_ff)) for o in range(len(wd))]


def moe_layer(x, w_router, experts, k, route="softmax", bias=None, shared=None,
              offset=None):
    """Whole layer on lists, token by token (tokens are independent)."""
    logits = matvec_rows(x, w_router)
    out = []
    for t, row in enumerate(logits):
        if offset is not None:
            row = [row[e] + offset[e] for e in range(len(row))]
        if route == "softmax":
            sel, g = route_softmax_all_renorm(row, k)
        else:
            sel, g = route_sigmoid_bias(row, k, bias)
        acc = [0.0] * len(x[t])
        for e, ge in zip(sel, g):
            y = swiglu(x[t], *experts[e])
            acc = [a + ge * v for a, v in zip(acc, y)]
        if shared is not None:
            ys = swiglu(x[t], *shared)
            acc = [a + v for a, v in zip(acc, ys)]
        out.append(acc)
    return out


def load_stats(logits, counts, k, alpha):
    """f_i = count_i / (T k), P_i = mean over tokens of softmax(logits_t)_i,
    aux = alpha * N * sum_i f_i P_i, by explicit loops."""
    T, N = len(logits), len(logits[0])
    P = [0.0] * N
    for t in range(T):
        m = max(logits[t])
        z = [math.exp(v - m) for v in logits[t]]
        tot = math.fsum(z)
        for i in range(N):
            P[i] += z[i] / tot / T
    f = [counts[i] / (T * k) for i in range(N)]
    return f, P, alpha * N * math.fsum(f[i] * P[i] for i in range(N))


def capacity_keep(idx, n_experts, cap):
    """First come, first served in token order then slot order: keep[t][i]."""
    used = [0] * n_experts
    keep = []
    for row in idx:
        kr = []
        for e in row:
            kr.append(used[e] < cap)
            used[e] += 1
        keep.append(kr)
    return keep


def group_limited(scores, k, n_groups, max_groups):
    """Enumerate every set of max_groups groups; a set's value is its sorted
    list of group maxima (float32) compared lexicographically, ties to the
    set of lower group indices; then the k best experts inside the winning
    set, ties to lower indices."""
    N = len(scores[0])
    gs = N // n_groups
    out = []
    for row in scores:
        r = [f32(v) for v in row]
        gmax = [max(r[g * gs:(g + 1) * gs]) for g in range(n_groups)]
        best = None
        for gset in itertools.combinations(range(n_groups), max_groups):
            key = (sorted((-gmax[g], g) for g in gset))
            if best is None or key < best[0]:
                best = (key, gset)
        allowed = [e for g in best[1] for e in range(g * gs, (g + 1) * gs)]
        out.append(sorted(allowed, key=lambda e: (-r[e], e))[:k])
    return out
