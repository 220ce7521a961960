"""The per-rank decomposition of the layer and the sum of row partials (oracle side).

Written without calling ``oracle.layer`` so the two can check each other:
this module uses einsum, the tanh form of the logistic function and a
log-sum-exp softmax where ``layer`` uses matmul, 1/(1+e^-z) and max-shifted
exponentials.

Sources: "Tensor Parallelism Fundamentals", section "Mechanics of Matrix
Slicing" (column-parallel: weight sliced by columns, input duplicated, each GPU
gets its slice of output columns; row-parallel: the column-parallel output is
fed directly in, the weight is sliced by rows, every GPU holds a partial sum
and the all-reduce adds the partials); "Tensor parallel scaling curves",
section "What tensor parallelism actually splits" (which projections are
column- and which row-split, owned heads, two sums per layer).

The all-reduce is replaced by a plain float64 sum of the t partials in rank
order; residual adds are applied once, after that sum.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np

from . import plan as _plan


def _f(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _norm(x, gamma, eps):
    x = _f(x)
    if gamma is None:
        return x
    inv = 1.0 / np.sqrt(np.einsum("mk,mk->m", x, x) / x.shape[1] + eps)
    return x * inv[:, None] * _f(gamma)[None, :]


def _silu(z):
    z = _f(z)
    return z * 0.5 * (1.0 + np.tanh(0.5 * z))


def _mm(a, w):
    return np.einsum("mk,kn->mn", _f(a), _f(w))


def column_shard(w, begin: int, count: int) -> np.ndarray:
    """Columns [begin, begin+count) of a logical [in, out] weight."""
    return np.asarray(w)[:, begin:begin + count]


def row_shard(w, begin: int, count: int) -> np.ndarray:
    """Rows [begin, begin+count) of a logical [in, out] weight."""
    return np.asarray(w)[begin:begin + count, :]


def sum_partials(partials: List[np.ndarray], residual=None) -> np.ndarray:
    """Sum in rank order (what the all-reduce returns), then the residual once."""
    acc = np.zeros_like(_f(partials[0]))
    for p in partials:
        acc = acc + _f(p)
    if residual is not None:
        acc = acc + _f(residual)
    return acc


def rank_mlp(x, w_gate, w_up, w_down, p: dict, gamma=None, eps: float = 1e-5) -> Dict[str, np.ndarray]:
    """One rank's MLP: column gate/up block, local SwiGLU, row-partial down."""
    b, c = p["inter_begin"], p["inter_cols"]
    u = _norm(x, gamma, eps)
    g = _mm(u, column_shard(w_gate, b, c))
    v = _mm(u, column_shard(w_up, b, c))
    a = _silu(g) * v
    partial = _mm(a, row_shard(w_down, b, c))
    return {"gate": g, "up": v, "a": a, "partial": partial}


def sharded_mlp(x, w_gate, w_up, w_down, t: int, gamma=None, eps: float = 1e-5) -> Dict[str, object]:
    H, I = np.shape(w_gate)
    desc = _plan.ModelDesc(hidden=H, intermediate=I)
    ranks = [rank_mlp(x, w_gate, w_up, w_down, _plan.rank_plan(desc, t, r), gamma, eps) for r in range(t)]
    return {"ranks": ranks, "sum": sum_partials([r["partial"] for r in ranks])}


def _attend(q_heads, keys, vals, d):
    """q_heads [G, d], keys/vals [S, d] -> [G, d], softmax by log-sum-exp."""
    s = np.einsum("gd,sd->gs", q_heads, keys) / np.sqrt(d)
    m = s.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(s - m).sum(axis=1, keepdims=True))
    return np.einsum("gs,sd->gd", np.exp(s - lse), vals)


def rank_attention(x, w_q, w_k, w_v, w_o, k_cache, v_cache, kv_len: int, n_q: int, n_kv: int, d: int,
                   p: dict, gamma=None, eps: float = 1e-5) -> Dict[str, np.ndarray]:
    """One rank's attention: owned q and kv heads, local cache append and attention, W_o partial.

    The caches passed in are unsharded [B, n_kv, capacity, d]; this rank reads and
    updates only its kv-head block.
    """
    qb, qn = p["q_head_begin"], p["q_heads"]
    kb, kn = p["kv_head_begin"], p["kv_heads"]
    u = _norm(x, gamma, eps)
    q = _mm(u, column_shard(w_q, qb * d, qn * d))
    k = _mm(u, column_shard(w_k, kb * d, kn * d))
    v = _mm(u, column_shard(w_v, kb * d, kn * d))
    B = q.shape[0]
    kc = _f(k_cache[:, kb:kb + kn]).copy()
    vc = _f(v_cache[:, kb:kb + kn]).copy()
    kc[:, :, kv_len - 1] = k.reshape(B, kn, d)
    vc[:, :, kv_len - 1] = v.reshape(B, kn, d)
    group = n_q // n_kv
    o = np.zeros((B, qn, d))
    for j in range(kn):                              # owned kv heads
        g_global = kb + j
        heads = [h - qb for h in range(qb, qb + qn) if h // group == g_global]
        for b in range(B):
            qh = q[b].reshape(qn, d)[heads]
            o[b, heads] = _attend(qh, kc[b, j, :kv_len], vc[b, j, :kv_len], d)
    o = o.reshape(B, qn * d)
    partial = _mm(o, row_shard(w_o, qb * d, qn * d))
    return {"q": q, "k": k, "v": v, "k_cache": kc, "v_cache": vc, "o": o, "partial": partial}


def rank_prefill_attention(q_rank, k_rank, v_rank, kv_len: int, n_q: int, n_kv: int, d: int,
                           p: dict) -> np.ndarray:
    """One rank's causal prefill attention on its owned heads.

    q_rank [B, S, q_heads * d] (the rank's q columns); k_rank, v_rank
    [B, kv_heads, capacity, d] (the rank's kv heads). Query i of the block sits
    at position kv_len - S + i and sees the first kv_len - S + i + 1 keys.
    """
    qb, qn = p["q_head_begin"], p["q_heads"]
    kb = p["kv_head_begin"]
    q = _f(q_rank)
    B, S = q.shape[0], q.shape[1]
    q = q.reshape(B, S, qn, d)
    group = n_q // n_kv
    o = np.zeros((B, S, qn, d))
    for b in range(B):
        for i in range(S):
            seen = kv_len - S + i + 1
            for hl in range(qn):
                j = (qb + hl) // group - kb           # local kv head
                o[b, i, hl] = _attend(q[b, i, hl][None, :], _f(k_rank[b, j, :seen]), _f(v_rank[b, j, :seen]), d)[0]
    return o.reshape(B, S, qn * d)


def rank_attention_prefill(x, w_q, w_k, w_v, w_o, k_cache, v_cache, kv_len: int, n_q: int, n_kv: int,
                           d: int, p: dict, gamma=None, eps: float = 1e-5) -> Dict[str, np.ndarray]:
    """One rank's attention stage for a block of S new tokens per sequence, x [B, S, H].

    Owned q and kv heads of every token; the block's k, v go into this rank's
    kv-head block of the (unsharded [B, n_kv, capacity, d]) caches at positions
    kv_len - S .. kv_len - 1; causal attention on the owned heads; W_o row
    partial [B, S, H].
    """
    x = _f(x)
    B, S, H = x.shape
    qb, qn = p["q_head_begin"], p["q_heads"]
    kb, kn = p["kv_head_begin"], p["kv_heads"]
    u = _norm(x.reshape(B * S, H), gamma, eps)
    q = _mm(u, column_shard(w_q, qb * d, qn * d)).reshape(B, S, qn * d)
    k = _mm(u, column_shard(w_k, kb * d, kn * d)).reshape(B, S, kn, d)
    v = _mm(u, column_shard(w_v, kb * d, kn * d)).reshape(B, S, kn, d)
    kc = _f(k_cache[:, kb:kb + kn]).copy()
    vc = _f(v_cache[:, kb:kb + kn]).copy()
    for i in range(S):
        kc[:, :, kv_len - S + i] = k[:, i]
        vc[:, :, kv_len - S + i] = v[:, i]
    o = rank_prefill_attention(q, kc, vc, kv_len, n_q, n_kv, d, p).reshape(B * S, qn * d)
    partial = _mm(o, row_shard(w_o, qb * d, qn * d)).reshape(B, S, H)
    return {"q": q, "k_cache": kc, "v_cache": vc, "o": o, "partial": partial}


def sharded_layer_prefill(x, w: Dict[str, Optional[np.ndarray]], k_cache, v_cache, kv_len: int, n_q: int,
                          n_kv: int, d: int, t: int, eps: float = 1e-5, residual: bool = True) -> Dict[str, object]:
    """All t ranks of the attention stage over a token block x [B, S, H], sum, then the MLP stage, sum."""
    x = _f(x)
    B, S, H = x.shape
    I = np.shape(w["w_gate"])[1]
    desc = _plan.ModelDesc(hidden=H, intermediate=I, n_q_heads=n_q, n_kv_heads=n_kv, head_dim=d)
    plans = [_plan.rank_plan(desc, t, r) for r in range(t)]
    attn = [rank_attention_prefill(x, w["w_q"], w["w_k"], w["w_v"], w["w_o"], k_cache, v_cache, kv_len,
                                   n_q, n_kv, d, p, w.get("gamma1"), eps) for p in plans]
    h = sum_partials([a["partial"] for a in attn], x if residual else None)
    h2 = h.reshape(B * S, H)
    mlp = [rank_mlp(h2, w["w_gate"], w["w_up"], w["w_down"], p, w.get("gamma2"), eps) for p in plans]
    out = sum_partials([m["partial"] for m in mlp], h2 if residual else None).reshape(B, S, H)
    return {"plans": plans, "attn": attn, "h": h, "mlp": mlp, "out": out}


def sharded_layer(x, w: Dict[str, Optional[np.ndarray]], k_cache, v_cache, kv_len: int, n_q: int,
                  n_kv: int, d: int, t: int, eps: float = 1e-5, residual: bool = True) -> Dict[str, object]:
    """All t ranks of the attention stage, sum, then all t ranks of the MLP stage, sum."""
    H = np.shape(x)[1]
    I = np.shape(w["w_gate"])[1]
    desc = _plan.ModelDesc(hidden=H, intermediate=I, n_q_heads=n_q, n_kv_heads=n_kv, head_dim=d)
    plans = [_plan.rank_plan(desc, t, r) for r in range(t)]
    attn = [rank_attention(x, w["w_q"], w["w_k"], w["w_v"], w["w_o"], k_cache, v_cache, kv_len,
                           n_q, n_kv, d, p, w.get("gamma1"), eps) for p in plans]
    h = sum_partials([a["partial"] for a in attn], x if residual else None)
    mlp = [rank_mlp(h, w["w_gate"], w["w_up"], w["w_down"], p, w.get("gamma2"), eps) for p in plans]
    out = sum_partials([m["partial"] for m in mlp], h if residual else None)
    return {"plans": plans, "attn": attn, "h": h, "mlp": mlp, "out": out}


def rank_moe(x, gamma, w_router, experts, gates, p: dict, eps: float = 1e-5) -> Dict[str, np.ndarray]:
    """One rank's share of a mixture-of-experts FFN: every expert's gate/up
    column block and down row block (the expert FFNs are sharded like the
    dense MLP), weighted by the routing gates [m, E] the router (replicated
    on every rank) produced, summed over the experts into one row partial."""
    b, c = p["inter_begin"], p["inter_cols"]
    u = _norm(x, gamma, eps)
    gates = _f(gates)
    partial = np.zeros((u.shape[0], np.shape(experts[0][2])[1]))
    acts = []
    for e, (wg, wu, wd) in enumerate(experts):
        g = _mm(u, column_shard(wg, b, c))
        v = _mm(u, column_shard(wu, b, c))
        a = _silu(g) * v * gates[:, e][:, None]
        acts.append(a)
        partial = partial + _mm(a, row_shard(wd, b, c))
    return {"a": np.concatenate(acts, axis=1), "partial": partial}
