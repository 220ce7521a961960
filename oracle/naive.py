"""Pure-Python loops for tiny shapes (oracle side), used to pin the numpy code.

Each function spells out one definition with explicit indices and ``math``
scalar functions, so a transposed operand or a wrong axis in the vectorised
oracle disagrees with it. Inputs are nested lists or numpy arrays; outputs are
nested Python lists of floats.
"""
from __future__ import annotations

import math


def matmul(a, w):
    """c[i][j] = sum_k a[i][k] * w[k][j]; w is logical [in, out]."""
    rows, inner, cols = len(a), len(w), len(w[0])
    out = []
    for i in range(rows):
        row = []
        for j in range(cols):
            s = 0.0
            for k in range(inner):
                s += float(a[i][k]) * float(w[k][j])
            row.append(s)
        out.append(row)
    return out


def rmsnorm(x, gamma, eps):
    out = []
    for row in x:
        n = len(row)
        ms = sum(float(v) * float(v) for v in row) / n
        r = 1.0 / math.sqrt(ms + eps)
        out.append([float(row[k]) * r * float(gamma[k]) for k in range(n)])
    return out


def silu(z):
    z = float(z)
    if z < -700.0:
        return 0.0 * z
    return z / (1.0 + math.exp(-z))


def mlp(x, w_gate, w_up, w_down, gamma=None, eps=1e-5):
    u = rmsnorm(x, gamma, eps) if gamma is not None else [[float(v) for v in r] for r in x]
    g = matmul(u, w_gate)
    v = matmul(u, w_up)
    a = [[silu(g[i][j]) * v[i][j] for j in range(len(g[0]))] for i in range(len(g))]
    return matmul(a, w_down)


def decode_attention(q, k_cache, v_cache, kv_len, n_q, n_kv, d):
    """q [B][n_q*d]; caches [B][n_kv][cap][d]; out [B][n_q*d]."""
    group = n_q // n_kv
    out = []
    for b in range(len(q)):
        row = []
        for h in range(n_q):
            g = h // group
            scores = []
            for j in range(kv_len):
                s = 0.0
                for e in range(d):
                    s += float(q[b][h * d + e]) * float(k_cache[b][g][j][e])
                scores.append(s / math.sqrt(d))
            mx = max(scores)
            w = [math.exp(s - mx) for s in scores]
            tot = sum(w)
            for e in range(d):
                acc = 0.0
                for j in range(kv_len):
                    acc += w[j] / tot * float(v_cache[b][g][j][e])
                row.append(acc)
        out.append(row)
    return out


def prefill_attention(q, k_cache, v_cache, kv_len, n_q, n_kv, d):
    """q [B][S][n_q*d] at positions kv_len-S..kv_len-1; caches [B][n_kv][cap][d]; out [B][S][n_q*d]."""
    group = n_q // n_kv
    out = []
    for b in range(len(q)):
        S = len(q[b])
        rows = []
        for i in range(S):
            pos = kv_len - S + i
            row = []
            for h in range(n_q):
                g = h // group
                scores = []
                for j in range(pos + 1):
                    s = 0.0
                    for e in range(d):
                        s += float(q[b][i][h * d + e]) * float(k_cache[b][g][j][e])
                    scores.append(s / math.sqrt(d))
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = sum(w)
                for e in range(d):
                    acc = 0.0
                    for j in range(pos + 1):
                        acc += w[j] / tot * float(v_cache[b][g][j][e])
                    row.append(acc)
            rows.append(row)
        out.append(rows)
    return out
