"""The unsharded layer in float64, written as its textbook definition (oracle side).

Data flow ("Tensor parallel scaling curves", section "What tensor parallelism
actually splits", and "Tensor Parallelism Fundamentals", section "Mechanics of
Matrix Slicing"): the attention block computes q, k, v = x @ W_q, x @ W_k,
x @ W_v, attends per head and projects with W_o; the MLP block applies gate and
up projections and a down projection. Weights are logical [in, out].

Readings the pages leave open:
- The nonlinearity between gate/up and down is SwiGLU: silu(x @ W_gate) *
  (x @ W_up), silu(z) = z * sigmoid(z) (Shazeer 2020, "GLU Variants Improve
  Transformer").
- RMSNorm is y = x * gamma / sqrt(mean(x^2) + eps) (Zhang & Sennrich 2019).
- Decode attention: one query per sequence, scores scaled by 1/sqrt(d), a
  softmax over the kv_len cached keys, no mask and no rotary embedding. The new
  token's k and v overwrite cache position kv_len - 1 before attending. Query
  head h reads kv head floor(h / (n_q / n_kv)) (grouped-query attention).
- Prefill attention: a block of S new tokens at positions kv_len - S ..
  kv_len - 1, whose k and v are already in the cache; the token at position p
  attends to positions 0..p (causal), with the same scale, grouping and no
  rotary embedding. A prompt from scratch is kv_len = S.
- The full layer is pre-norm with residual adds: h = x + attn(norm1(x)),
  out = h + mlp(norm2(h)); ``residual=False`` gives the pages' literal flow.
- No biases.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def rmsnorm(x, gamma, eps: float) -> np.ndarray:
    """x * gamma / sqrt(mean over the last axis of x^2 + eps)."""
    x = f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * f64(gamma)


def sigmoid(z) -> np.ndarray:
    z = f64(z)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z) -> np.ndarray:
    """z * sigmoid(z)."""
    z = f64(z)
    return z * sigmoid(z)


def swiglu(gate, up) -> np.ndarray:
    """silu(gate) * up."""
    return silu(gate) * f64(up)


def linear(x, w) -> np.ndarray:
    """x @ W with W logical [in, out]."""
    return f64(x) @ f64(w)


def mlp_block(x, w_gate, w_up, w_down, gamma=None, eps: float = 1e-5) -> Dict[str, np.ndarray]:
    """Optional RMSNorm, then SwiGLU MLP. Returns every intermediate."""
    u = rmsnorm(x, gamma, eps) if gamma is not None else f64(x)
    g = linear(u, w_gate)
    v = linear(u, w_up)
    a = swiglu(g, v)
    y = linear(a, w_down)
    return {"u": u, "gate": g, "up": v, "a": a, "y": y}


def softmax(s) -> np.ndarray:
    s = f64(s)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def decode_attention(q, k_cache, v_cache, kv_len: int, n_q: int, n_kv: int, d: int) -> np.ndarray:
    """Grouped-query decode attention.

    q [B, n_q * d]; caches [B, n_kv, capacity, d]; attends to positions 0..kv_len-1.
    Returns [B, n_q * d] in head-major order.
    """
    q = f64(q).reshape(q.shape[0], n_q, d)
    B = q.shape[0]
    group = n_q // n_kv
    out = np.zeros((B, n_q, d))
    scale = 1.0 / np.sqrt(d)
    for b in range(B):
        for h in range(n_q):
            g = h // group
            keys = f64(k_cache[b, g, :kv_len])          # [kv_len, d]
            vals = f64(v_cache[b, g, :kv_len])
            p = softmax((keys @ q[b, h]) * scale)       # [kv_len]
            out[b, h] = p @ vals
    return out.reshape(B, n_q * d)


def prefill_attention(q, k_cache, v_cache, kv_len: int, n_q: int, n_kv: int, d: int) -> np.ndarray:
    """Causal grouped-query attention for a block of new tokens.

    q [B, S, n_q * d] for the tokens at positions kv_len - S .. kv_len - 1;
    caches [B, n_kv, capacity, d] hold k, v for positions 0..kv_len-1. The
    token at position p attends to positions 0..p. Returns [B, S, n_q * d].
    """
    q = f64(q)
    B, S = q.shape[0], q.shape[1]
    q = q.reshape(B, S, n_q, d)
    group = n_q // n_kv
    scale = 1.0 / np.sqrt(d)
    pos = (kv_len - S) + np.arange(S)                    # position of each query
    allowed = np.arange(kv_len)[None, :] <= pos[:, None]  # [S, kv_len]
    out = np.zeros((B, S, n_q, d))
    for b in range(B):
        for h in range(n_q):
            g = h // group
            keys = f64(k_cache[b, g, :kv_len])
            vals = f64(v_cache[b, g, :kv_len])
            s = np.where(allowed, (q[b, :, h] @ keys.T) * scale, -np.inf)
            out[b, :, h] = softmax(s) @ vals
    return out.reshape(B, S, n_q * d)


def append_kv(k_cache, v_cache, k_new, v_new, kv_len: int, n_kv: int, d: int):
    """Copies of the caches with the new token's k, v [B, n_kv * d] at position kv_len - 1."""
    kc = f64(k_cache).copy()
    vc = f64(v_cache).copy()
    B = kc.shape[0]
    kc[:, :, kv_len - 1, :] = f64(k_new).reshape(B, n_kv, d)
    vc[:, :, kv_len - 1, :] = f64(v_new).reshape(B, n_kv, d)
    return kc, vc


def attention_block(x, w_q, w_k, w_v, w_o, k_cache, v_cache, kv_len: int, n_q: int, n_kv: int,
                    d: int, gamma=None, eps: float = 1e-5) -> Dict[str, np.ndarray]:
    """Optional RMSNorm, QKV projections, KV append, decode attention, output projection."""
    u = rmsnorm(x, gamma, eps) if gamma is not None else f64(x)
    q = linear(u, w_q)
    k = linear(u, w_k)
    v = linear(u, w_v)
    kc, vc = append_kv(k_cache, v_cache, k, v, kv_len, n_kv, d)
    o = decode_attention(q, kc, vc, kv_len, n_q, n_kv, d)
    y = linear(o, w_o)
    return {"u": u, "q": q, "k": k, "v": v, "k_cache": kc, "v_cache": vc, "o": o, "y": y}


def append_kv_block(k_cache, v_cache, k_new, v_new, kv_len: int, n_kv: int, d: int):
    """Copies of the caches with a block's k, v [B, S, n_kv * d] at positions kv_len - S .. kv_len - 1."""
    kc = f64(k_cache).copy()
    vc = f64(v_cache).copy()
    B, S = np.shape(k_new)[0], np.shape(k_new)[1]
    kc[:, :, kv_len - S:kv_len, :] = f64(k_new).reshape(B, S, n_kv, d).transpose(0, 2, 1, 3)
    vc[:, :, kv_len - S:kv_len, :] = f64(v_new).reshape(B, S, n_kv, d).transpose(0, 2, 1, 3)
    return kc, vc


def attention_block_prefill(x, w_q, w_k, w_v, w_o, k_cache, v_cache, kv_len: int, n_q: int, n_kv: int,
                            d: int, gamma=None, eps: float = 1e-5) -> Dict[str, np.ndarray]:
    """The attention block for a block of S new tokens per sequence, x [B, S, H].

    Optional RMSNorm and the QKV projections of every token, the block's k, v
    written to cache positions kv_len - S .. kv_len - 1, causal prefill
    attention, output projection. Returns y [B, S, H] (and the pieces).
    """
    x = f64(x)
    B, S, H = x.shape
    u = rmsnorm(x.reshape(B * S, H), gamma, eps) if gamma is not None else x.reshape(B * S, H)
    q = linear(u, w_q).reshape(B, S, -1)
    k = linear(u, w_k).reshape(B, S, -1)
    v = linear(u, w_v).reshape(B, S, -1)
    kc, vc = append_kv_block(k_cache, v_cache, k, v, kv_len, n_kv, d)
    o = prefill_attention(q, kc, vc, kv_len, n_q, n_kv, d)
    y = linear(o.reshape(B * S, -1), w_o).reshape(B, S, H)
    return {"u": u, "q": q, "k": k, "v": v, "k_cache": kc, "v_cache": vc, "o": o, "y": y}


def layer_prefill(x, w: Dict[str, np.ndarray], k_cache, v_cache, kv_len: int, n_q: int, n_kv: int, d: int,
                  eps: float = 1e-5, residual: bool = True) -> Dict[str, np.ndarray]:
    """The layer over a block of S new tokens per sequence, x [B, S, H]: attention block, then MLP block."""
    x = f64(x)
    B, S, H = x.shape
    attn = attention_block_prefill(x, w["w_q"], w["w_k"], w["w_v"], w["w_o"], k_cache, v_cache, kv_len,
                                   n_q, n_kv, d, w.get("gamma1"), eps)
    h = x + attn["y"] if residual else attn["y"]
    mlp = mlp_block(h.reshape(B * S, H), w["w_gate"], w["w_up"], w["w_down"], w.get("gamma2"), eps)
    y = mlp["y"].reshape(B, S, H)
    out = h + y if residual else y
    return {"attn": attn, "h": h, "mlp": mlp, "out": out}


def layer(x, w: Dict[str, np.ndarray], k_cache, v_cache, kv_len: int, n_q: int, n_kv: int, d: int,
          eps: float = 1e-5, residual: bool = True) -> Dict[str, np.ndarray]:
    """Attention block then MLP block.

    ``w`` holds gamma1, w_q, w_k, w_v, w_o, gamma2, w_gate, w_up, w_down (gammas may be None).
    With ``residual`` the block is pre-norm with residual adds; without it, the MLP
    consumes the attention output directly, as in the pages' pseudocode.
    """
    attn = attention_block(x, w["w_q"], w["w_k"], w["w_v"], w["w_o"], k_cache, v_cache, kv_len,
                           n_q, n_kv, d, w.get("gamma1"), eps)
    h = f64(x) + attn["y"] if residual else attn["y"]
    mlp = mlp_block(h, w["w_gate"], w["w_up"], w["w_down"], w.get("gamma2"), eps)
    out = h + mlp["y"] if residual else mlp["y"]
    return {"attn": attn, "h": h, "mlp": mlp, "out": out}


def attn_proj_block(x, attn_in, w_q, w_k, w_v, w_o) -> Dict[str, np.ndarray]:
    """QKV projections of x and W_o applied to a given attention output (no attention between)."""
    return {"q": linear(x, w_q), "k": linear(x, w_k), "v": linear(x, w_v), "y": linear(attn_in, w_o)}


def maybe(a: Optional[np.ndarray]) -> Optional[np.ndarray]:
    return None if a is None else f64(a)


def moe_route(logits, k: int) -> np.ndarray:
    """Router gates [m, E] from logits [m, E]: the k largest logits of a token
    (ties to the lower expert index) get softmax weights over those k alone,
    the other experts 0. (Mixtral-style top-k routing; the softmax over the
    selected logits equals a softmax over all experts renormalised on the top k.)
    """
    logits = f64(logits)
    m, E = logits.shape
    gates = np.zeros((m, E))
    for t in range(m):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        sel = logits[t, order]
        p = np.exp(sel - sel.max())
        gates[t, order] = p / p.sum()
    return gates


def moe_block(x, gamma, w_router, experts, k: int, eps: float = 1e-5, gates=None) -> Dict[str, np.ndarray]:
    """Mixture-of-experts FFN: u = RMSNorm(x); gates from u @ W_router [H, E];
    y = sum_e gate[:, e] * (swiglu(u @ W_gate_e, u @ W_up_e) @ W_down_e).

    ``experts`` is a list of (w_gate [H, I], w_up [H, I], w_down [I, H]).
    ``gates`` may be given to take the routing decision elsewhere (for
    instance on logits computed in another precision).
    """
    u = rmsnorm(x, gamma, eps) if gamma is not None else f64(x)
    logits = linear(u, w_router)
    if gates is None:
        gates = moe_route(logits, k)
    y = np.zeros((u.shape[0], np.shape(experts[0][2])[1]))
    for e, (wg, wu, wd) in enumerate(experts):
        y += gates[:, e:e + 1] * linear(swiglu(linear(u, wg), linear(u, wu)), wd)
    return {"u": u, "logits": logits, "gates": gates, "y": y}
