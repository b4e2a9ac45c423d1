"""Pure-Python brute force of the compressed-sparse-attention chain for tiny shapes.

No numpy arithmetic: plain floats, math.exp / math.sqrt and explicit loops, so
that it shares no vectorised expression with the oracle it cross-checks.
Used only by the oracle self-tests.
"""
from __future__ import annotations

import math


def softmax_weighted(xs, ls):
    """xs, ls: lists of w rows (lists of D floats). Per-channel softmax over rows."""
    d = len(xs[0])
    out = []
    for c in range(d):
        m = max(l[c] for l in ls)
        es = [math.exp(l[c] - m) for l in ls]
        den = sum(es)
        out.append(sum(e * x[c] for e, x in zip(es, xs)) / den)
    return out


def rmsnorm(z, gamma, eps):
    ms = sum(v * v for v in z) / len(z)
    r = 1.0 / math.sqrt(ms + eps)
    return [v * r * g for v, g in zip(z, gamma)]


def rotate(y, cs, rdims, sign):
    """sign=+1 RoPE, sign=-1 inverse. cs: list of (cos, sin) pairs."""
    y = list(y)
    d = len(y)
    base = d - rdims
    for j in range(rdims // 2):
        c, s = cs[j]
        u, v = y[base + 2 * j], y[base + 2 * j + 1]
        y[base + 2 * j] = u * c - sign * v * s
        y[base + 2 * j + 1] = sign * u * s + v * c
    return y


def compress(x_seq, g_seq, ratio, window, gamma, eps, table, rdims):
    """All entries of a raw sequence. x_seq[j] = row, g_seq[j][role] = logit row."""
    n = len(x_seq)
    out = []
    i = 0
    while ratio * i + window - 1 <= n - 1:
        xs = [x_seq[ratio * i + t] for t in range(window)]
        ls = [g_seq[ratio * i + t][t // ratio] for t in range(window)]
        z = softmax_weighted(xs, ls)
        y = rmsnorm(z, gamma, eps)
        out.append(rotate(y, table[ratio * i], rdims, +1))
        i += 1
    return out


def dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def wrelu_score(q_heads, w, k):
    return sum(wh * max(0.0, dot(qh, k)) for qh, wh in zip(q_heads, w))


def topk_sorted(scores, k):
    order = sorted(range(len(scores)), key=lambda i: (-scores[i], i))
    return sorted(order[:k])


def attend(q_heads, keys, scale):
    outs, lses = [], []
    for qh in q_heads:
        lg = [scale * dot(qh, kk) for kk in keys]
        m = max(lg)
        es = [math.exp(v - m) for v in lg]
        den = sum(es)
        outs.append([sum(e * kk[c] for e, kk in zip(es, keys)) / den for c in range(len(keys[0]))])
        lses.append(m + math.log(den))
    return outs, lses
