"""Pins of the oracle, written as check functions over the functions they pin.

Each ``pin_*`` raises AssertionError when the function given to it disagrees
with what the pages or the mathematics fix. ``test_oracle_pins`` runs them on
the oracle as it is; ``test_oracle_mutations`` runs them on copies of the
oracle with a planted mistake and expects at least one to fail. Nothing here
recomputes a result by the oracle's own formula: every expected value is a
printed number, a closed form evaluated by hand, an identity, or a brute-force
loop from ``oracle.naive``.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import workloads as W
from oracle import naive

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
GiB = 1 << 30


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def relerr(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (scale if scale > 0 else 1.0))


# ---------------------------------------------------------------- planner

def pin_kv_worked_example(kv_elements_per_sequence, kv_bytes_per_gpu):
    g = golden("kv_cache_worked_example.json")
    e = kv_elements_per_sequence(g["n_layers"], g["n_kv_heads"], g["head_dim"], g["seq_len"])
    assert e == g["elements_per_sequence"], e
    assert e * g["bytes_per_element"] == g["GiB_per_sequence"] * GiB
    whole = kv_bytes_per_gpu(g["n_layers"], g["n_kv_heads"], g["head_dim"], g["seq_len"],
                             g["bytes_per_element"], g["batch"], 1)
    assert whole == g["GiB_whole_batch"] * GiB, whole
    per = kv_bytes_per_gpu(g["n_layers"], g["n_kv_heads"], g["head_dim"], g["seq_len"],
                           g["bytes_per_element"], g["batch"], g["t"])
    assert per == g["GiB_per_gpu"] * GiB, per


def pin_weight_footprint(weight_bytes_per_gpu):
    g = golden("weight_footprint.json")
    total = g["parameters"] * g["bytes_per_element"]
    assert total == g["total_GB"] * 10**9
    assert weight_bytes_per_gpu(total, g["t"]) == g["per_gpu_GB"] * 10**9


def pin_head_blocks(rank_plan, ModelDesc):
    """Owned blocks are heads[rank*h : (rank+1)*h] and partition every head, kv head and column."""
    for n_q, n_kv, inter, t in [(64, 8, 28672, 8), (64, 8, 28672, 4), (32, 8, 14336, 2),
                                (8, 8, 64, 8), (6, 2, 12, 2), (4, 4, 8, 1), (12, 3, 9, 3)]:
        desc = ModelDesc(hidden=16, intermediate=inter, n_q_heads=n_q, n_kv_heads=n_kv, head_dim=4)
        seen_q, seen_kv, seen_i = [], [], []
        for r in range(t):
            p = rank_plan(desc, t, r)
            h = n_q // t
            assert (p["q_head_begin"], p["q_heads"]) == (r * h, h)
            seen_q += list(range(p["q_head_begin"], p["q_head_begin"] + p["q_heads"]))
            seen_kv += list(range(p["kv_head_begin"], p["kv_head_begin"] + p["kv_heads"]))
            seen_i += list(range(p["inter_begin"], p["inter_begin"] + p["inter_cols"]))
            # every owned q head's kv head (grouped-query mapping) is owned by the same rank
            grp = n_q // n_kv
            for qh in range(p["q_head_begin"], p["q_head_begin"] + p["q_heads"]):
                assert p["kv_head_begin"] <= qh // grp < p["kv_head_begin"] + p["kv_heads"]
        assert seen_q == list(range(n_q)) and seen_kv == list(range(n_kv)) and seen_i == list(range(inter))


def pin_workload_shapes(rank_plan, ModelDesc):
    """Per-rank shapes stated in the workload definitions of the five measured workloads."""
    # tiny MLP, t=2: gate/up 256x512 each, down 512x256
    p = rank_plan(ModelDesc(hidden=256, intermediate=1024), 2, 1)
    assert (p["inter_begin"], p["inter_cols"]) == (512, 512)
    # Llama-3-8B-shaped MLP, t=4: gate/up 4096x3584 each, down 3584x4096
    p = rank_plan(ModelDesc(hidden=4096, intermediate=14336), 4, 3)
    assert (p["inter_begin"], p["inter_cols"]) == (3 * 3584, 3584)
    # 70B-shaped attention projections, t=4: W_qkv 8192x2560 (16 q + 2 kv heads), W_o 2048x8192
    p = rank_plan(ModelDesc(hidden=8192, n_q_heads=64, n_kv_heads=8, head_dim=128), 4, 2)
    assert (p["q_heads"], p["kv_heads"], p["qkv_cols"], p["o_rows"]) == (16, 2, 2560, 2048)
    # 70B-shaped MLP prefill, t=4: gate/up 8192x7168, down 7168x8192
    p = rank_plan(ModelDesc(hidden=8192, intermediate=28672), 4, 0)
    assert p["inter_cols"] == 7168
    # 70B-shaped full layer, t=8: 8 q heads, 1 kv head, MLP 8192->3584
    desc = ModelDesc(hidden=8192, intermediate=28672, n_q_heads=64, n_kv_heads=8, head_dim=128,
                     n_layers=1, seq_len=8192, batch=16, bytes_per_elem=2)
    p = rank_plan(desc, 8, 7)
    assert (p["q_heads"], p["kv_heads"], p["qkv_cols"], p["o_rows"], p["inter_cols"]) == (8, 1, 1280, 1024, 3584)
    # one layer's KV at batch 16, seq 8192, bf16, t=8: 2*8*128*8192*2*16/8 bytes
    assert p["kv_bytes_rank"] == 67_108_864
    # 70B layer: 150,994,944 attention + 704,643,072 MLP weights, split evenly over 8 ranks
    assert sum(rank_plan(desc, 8, r)["weight_elems"] for r in range(8)) == 855_638_016
    assert p["weight_elems"] == 855_638_016 // 8


def pin_layer_weight_elements(layer_weight_elements, rank_plan, ModelDesc):
    """One layer's projection weights: hand-evaluated counts for two public shapes, and the rank
    shards partitioning them (no kv-head replication)."""
    # 70B shape: 8192*(64+2*8)*128 (QKV) + 64*128*8192 (W_o) + 3*8192*28672 (gate, up, down)
    d70 = ModelDesc(hidden=8192, intermediate=28672, n_q_heads=64, n_kv_heads=8, head_dim=128)
    assert layer_weight_elements(d70) == 855_638_016
    # Llama-3-8B shape: 4096*(32+2*8)*128 + 32*128*4096 + 3*4096*14336
    d8 = ModelDesc(hidden=4096, intermediate=14336, n_q_heads=32, n_kv_heads=8, head_dim=128)
    assert layer_weight_elements(d8) == 218_103_808
    # an MLP-only block has no attention weights
    assert layer_weight_elements(ModelDesc(hidden=256, intermediate=1024)) == 3 * 256 * 1024
    for desc in (d70, d8):
        for t in (1, 2, 4, 8):
            assert sum(rank_plan(desc, t, r)["weight_elems"] for r in range(t)) == layer_weight_elements(desc)


def pin_plan_errors(rank_plan, ModelDesc, PlanError):
    bad = [
        (ModelDesc(hidden=8, intermediate=8), 0, 0, "RANK"),
        (ModelDesc(hidden=8, intermediate=8), 9, 0, "RANK"),
        (ModelDesc(hidden=8, intermediate=8), 2, 2, "RANK"),
        (ModelDesc(hidden=8, intermediate=8), 2, -1, "RANK"),
        (ModelDesc(hidden=8, intermediate=9), 2, 0, "INDIVISIBLE"),
        (ModelDesc(hidden=8, n_q_heads=64, n_kv_heads=8, head_dim=4), 3, 0, "INDIVISIBLE"),
        (ModelDesc(hidden=8, n_q_heads=6, n_kv_heads=4, head_dim=4), 2, 0, "INDIVISIBLE"),
        (ModelDesc(hidden=8, n_q_heads=12, n_kv_heads=4, head_dim=4), 6, 0, "INDIVISIBLE"),
        (ModelDesc(hidden=8, n_q_heads=8, n_kv_heads=2, head_dim=4), 3, 0, "INDIVISIBLE"),
        (ModelDesc(hidden=0, intermediate=8), 1, 0, "SHAPE"),
        (ModelDesc(hidden=8, n_q_heads=8, n_kv_heads=0, head_dim=4), 1, 0, "SHAPE"),
    ]
    for desc, t, r, kind in bad:
        try:
            rank_plan(desc, t, r)
        except PlanError as e:
            assert e.kind == kind, (desc, t, r, e.kind)
        else:
            raise AssertionError(f"accepted {desc} t={t} rank={r}")


# ---------------------------------------------------------------- elementwise

def pin_silu(silu):
    z = np.linspace(-20.0, 20.0, 401)
    assert float(silu(np.array(0.0))) == 0.0
    # silu(z) - silu(-z) = z * (sigmoid(z) + sigmoid(-z)) = z
    assert np.max(np.abs(silu(z) - silu(-z) - z)) < 1e-12
    # silu(1) = 1/(1+e^-1), evaluated by hand
    assert abs(float(silu(np.array(1.0))) - 0.7310585786300049) < 1e-15
    # silu(-1) = -e^-1/(1+e^-1)
    assert abs(float(silu(np.array(-1.0))) + 0.2689414213699951) < 1e-15
    big = silu(np.array([100.0, -100.0, 1000.0, -1000.0]))
    assert np.all(np.isfinite(big))
    assert abs(big[0] - 100.0) < 1e-12 and abs(big[1]) < 1e-40
    assert big[2] == 1000.0 and big[3] == 0.0


def pin_rmsnorm(rmsnorm):
    # [3, 4]: mean square 12.5; values 3/sqrt(12.5), 4/sqrt(12.5)
    y = rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 1.0]), 0.0)
    assert np.allclose(y, [[0.848528137423857, 1.131370849898476]], rtol=0, atol=1e-15)
    # constant vector c: gamma * c / sqrt(c^2 + eps)
    c, eps = 0.5, 1e-5
    y = rmsnorm(np.full((1, 6), c), np.arange(1.0, 7.0), eps)
    assert np.allclose(y, np.arange(1.0, 7.0) * c / math.sqrt(c * c + eps), rtol=0, atol=1e-14)
    # rows are normalised independently and scale-invariant when eps = 0
    x = W.normal(99, 0, (3, 16)).astype(np.float64)
    g = W.normal(99, 1, (16,)).astype(np.float64)
    y1 = rmsnorm(x, g, 0.0)
    y2 = rmsnorm(x * np.array([[2.0], [0.25], [7.0]]), g, 0.0)
    assert np.max(np.abs(y1 - y2)) < 1e-13
    assert np.max(np.abs(rmsnorm(x[1:2], g, 0.0) - y1[1:2])) < 1e-15
    # mean of (y/gamma)^2 is 1 when eps = 0
    assert np.max(np.abs(np.mean((y1 / g) ** 2, axis=1) - 1.0)) < 1e-13


# ---------------------------------------------------------------- blocks vs brute force

def tiny_mlp(seed=7, m=3, H=8, I=12, gamma=True):
    d = W.mlp_inputs(seed, H, I, m, "f32", "random" if gamma else None)
    return d


def pin_mlp_vs_naive(mlp_block):
    for gamma in (False, True):
        d = tiny_mlp(gamma=gamma)
        ref = naive.mlp(d["x"], d["w_gate"], d["w_up"], d["w_down"], d.get("gamma"), 1e-5)
        got = mlp_block(d["x"], d["w_gate"], d["w_up"], d["w_down"], d.get("gamma"), 1e-5)["y"]
        assert relerr(got, ref) < 1e-13, relerr(got, ref)


def pin_attn_proj_block(attn_proj_block):
    """QKV projections of x and W_o applied to a separate attention output, against the pure-Python
    product. x and the attention output have the same shape but different values, and W_k, W_v differ,
    so feeding x to W_o or swapping K and V disagrees with the loop."""
    x = W.normal(71, 0, (3, 8))
    attn_in = W.normal(71, 1, (3, 8))
    w_q = W.normal(71, 2, (8, 8), 0.5)
    w_k = W.normal(71, 3, (8, 4), 0.5)
    w_v = W.normal(71, 4, (8, 4), 0.5)
    w_o = W.normal(71, 5, (8, 8), 0.5)
    got = attn_proj_block(x, attn_in, w_q, w_k, w_v, w_o)
    for name, a, w in (("q", x, w_q), ("k", x, w_k), ("v", x, w_v), ("y", attn_in, w_o)):
        ref = naive.matmul(a, w)
        assert relerr(got[name], ref) < 1e-14, name


def tiny_attention(seed=11, B=2, H=12, n_q=4, n_kv=2, d=3, cap=6):
    return W.attention_inputs(seed, H, n_q, n_kv, d, B, cap, "f32", "random")


def pin_attention_vs_naive(decode_attention):
    for n_q, n_kv in [(4, 2), (4, 4), (6, 1)]:
        a = tiny_attention(n_q=n_q, n_kv=n_kv)
        q = W.normal(12, 0, (2, n_q * 3))
        for kv_len in (1, 4, 6):
            ref = naive.decode_attention(q, a["k_cache"], a["v_cache"], kv_len, n_q, n_kv, 3)
            got = decode_attention(q, a["k_cache"], a["v_cache"], kv_len, n_q, n_kv, 3)
            assert relerr(got, ref) < 1e-13, (n_q, n_kv, kv_len)


def pin_attention_special_cases(decode_attention):
    B, n_q, n_kv, d, cap = 2, 4, 2, 5, 7
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, n_q * d))
    K = rng.standard_normal((B, n_kv, cap, d))
    V = rng.standard_normal((B, n_kv, cap, d))
    # kv_len = 1: the output is v_0 of the head's group
    o = decode_attention(q, K, V, 1, n_q, n_kv, d).reshape(B, n_q, d)
    for h in range(n_q):
        assert np.allclose(o[:, h], V[:, h // 2, 0], rtol=0, atol=1e-15)
    # identical keys: uniform weights, the mean of the attended values
    Kc = np.repeat(K[:, :, :1], cap, axis=2)
    o = decode_attention(q, Kc, V, 5, n_q, n_kv, d).reshape(B, n_q, d)
    for h in range(n_q):
        assert np.allclose(o[:, h], V[:, h // 2, :5].mean(axis=1), rtol=0, atol=1e-14)
    # one dominant score: that key's value
    qd = np.zeros((B, n_q * d)); qd[:, 0::d] = 1.0          # q_h = e_0 for every head
    Kd = np.zeros((B, n_kv, cap, d)); Kd[:, :, 3, 0] = 400.0
    o = decode_attention(qd, Kd, V, 6, n_q, n_kv, d).reshape(B, n_q, d)
    for h in range(n_q):
        assert np.allclose(o[:, h], V[:, h // 2, 3], rtol=0, atol=1e-12)
    # grouped-query mapping: values constant per kv head g equal g + 1
    Vg = np.zeros((B, n_kv, cap, d))
    for g in range(n_kv):
        Vg[:, g] = g + 1.0
    o = decode_attention(q, K, Vg, cap, n_q, n_kv, d).reshape(B, n_q, d)
    assert np.allclose(o[:, 0], 1.0) and np.allclose(o[:, 1], 1.0)
    assert np.allclose(o[:, 2], 2.0) and np.allclose(o[:, 3], 2.0)
    # positions at and beyond kv_len are never read
    Kx, Vx = K.copy(), V.copy()
    Kx[:, :, 4:] = np.nan; Vx[:, :, 4:] = np.nan
    assert np.all(np.isfinite(decode_attention(q, Kx, Vx, 4, n_q, n_kv, d)))
    # the softmax weights sum to one: with V = 1 everywhere the output is 1
    o = decode_attention(q, K, np.ones_like(V), cap, n_q, n_kv, d)
    assert np.max(np.abs(o - 1.0)) < 1e-14


def pin_prefill_attention(prefill_attention, decode_attention):
    """Causal prefill attention: brute force on tiny inputs, the first token's
    output is its own value, the last row is decode attention over the same
    keys, identical keys give running means, and a chunk of the block equals
    the same rows of the whole block."""
    B, n_q, n_kv, d, cap = 2, 4, 2, 3, 9
    rng = np.random.default_rng(21)
    K = rng.standard_normal((B, n_kv, cap, d))
    V = rng.standard_normal((B, n_kv, cap, d))
    for S, kv_len in [(1, 1), (3, 3), (4, 6), (5, 9)]:
        q = rng.standard_normal((B, S, n_q * d))
        ref = np.array(naive.prefill_attention(q.tolist(), K.tolist(), V.tolist(), kv_len, n_q, n_kv, d))
        got = prefill_attention(q, K, V, kv_len, n_q, n_kv, d)
        assert relerr(got, ref) < 1e-13, (S, kv_len)
        # the last query attends to every key: decode attention
        last = decode_attention(q[:, -1], K, V, kv_len, n_q, n_kv, d)
        assert relerr(got[:, -1], last) < 1e-13, (S, kv_len)
    # a prompt from scratch: token 0 sees only itself
    S = 6
    q = rng.standard_normal((B, S, n_q * d))
    o = prefill_attention(q, K, V, S, n_q, n_kv, d).reshape(B, S, n_q, d)
    for h in range(n_q):
        assert np.allclose(o[:, 0, h], V[:, h // 2, 0], rtol=0, atol=1e-15)
    # identical keys: the token at position p averages values 0..p
    Kc = np.repeat(K[:, :, :1], cap, axis=2)
    o = prefill_attention(q, Kc, V, S, n_q, n_kv, d).reshape(B, S, n_q, d)
    for i in range(S):
        for h in range(n_q):
            assert np.allclose(o[:, i, h], V[:, h // 2, :i + 1].mean(axis=1), rtol=0, atol=1e-14)
    # positions after a query are never read: poison them for the first rows
    Kx, Vx = K.copy(), V.copy()
    Kx[:, :, 3:] = np.nan; Vx[:, :, 3:] = np.nan
    o = prefill_attention(q[:, :3], Kx, Vx, 3, n_q, n_kv, d)
    assert np.all(np.isfinite(o))
    # chunked prefill: the last 2 rows of a 6-token block, given the same caches
    full = prefill_attention(q, K, V, S, n_q, n_kv, d)
    part = prefill_attention(q[:, 4:], K, V, S, n_q, n_kv, d)
    assert relerr(part, full[:, 4:]) < 1e-14


def pin_rank_prefill(rank_prefill_attention, prefill_attention, rank_plan, ModelDesc):
    """Each rank's owned heads, from its own kv heads, equal the unsharded heads."""
    B, S, n_q, n_kv, d, cap, kv_len = 2, 4, 8, 4, 3, 7, 6
    rng = np.random.default_rng(22)
    q = rng.standard_normal((B, S, n_q * d))
    K = rng.standard_normal((B, n_kv, cap, d))
    V = rng.standard_normal((B, n_kv, cap, d))
    full = prefill_attention(q, K, V, kv_len, n_q, n_kv, d)
    for t in (1, 2, 4):
        desc = ModelDesc(hidden=n_q * d, intermediate=0, n_q_heads=n_q, n_kv_heads=n_kv, head_dim=d)
        for r in range(t):
            p = rank_plan(desc, t, r)
            qs = slice(p["q_head_begin"] * d, (p["q_head_begin"] + p["q_heads"]) * d)
            ks = slice(p["kv_head_begin"], p["kv_head_begin"] + p["kv_heads"])
            got = rank_prefill_attention(q[:, :, qs], K[:, ks], V[:, ks], kv_len, n_q, n_kv, d, p)
            assert relerr(got, full[:, :, qs]) < 1e-13, (t, r)


# ---------------------------------------------------------------- decomposition invariants

def pin_column_concat_naive(column_shard, rank_plan, ModelDesc):
    """Column shards, multiplied with the same k order, concatenate bitwise to the whole."""
    d = tiny_mlp(m=2, H=6, I=8, gamma=False)
    full = naive.matmul(d["x"], d["w_gate"])
    for t in (1, 2, 4, 8):
        parts = []
        for r in range(t):
            p = rank_plan(ModelDesc(hidden=6, intermediate=8), t, r)
            parts.append(np.array(naive.matmul(d["x"], column_shard(d["w_gate"], p["inter_begin"], p["inter_cols"]))))
        assert np.array_equal(np.concatenate(parts, axis=1), np.array(full)), t


def pin_row_partials_sum(row_shard, sum_partials, rank_plan, ModelDesc):
    """Row partials sum to the whole within the float64 dot-product error bound."""
    H, I, m = 32, 64, 3
    d = W.mlp_inputs(21, H, I, m, "f32")
    a = W.normal(21, 50, (m, I)).astype(np.float64)
    whole = np.array(naive.matmul(a, d["w_down"]))
    for t in (1, 2, 4, 8):
        parts = []
        for r in range(t):
            p = rank_plan(ModelDesc(hidden=H, intermediate=I), t, r)
            b, c = p["inter_begin"], p["inter_cols"]
            parts.append(np.array(naive.matmul(a[:, b:b + c], row_shard(d["w_down"], b, c))))
        s = sum_partials(parts)
        bound = I * 2.0 ** -53 * np.max(np.abs(a) @ np.abs(d["w_down"].astype(np.float64)))
        assert np.max(np.abs(s - whole)) <= 4 * bound, t
        if t == 1:
            assert np.array_equal(s, whole)
        # the order of the partials changes the sum by no more than rounding
        assert np.max(np.abs(sum_partials(parts[::-1]) - s)) <= 4 * bound


def pin_sharded_mlp(sharded_mlp, mlp_block):
    d = W.mlp_inputs(31, 64, 256, 5, "f32", "random")
    ref = mlp_block(d["x"], d["w_gate"], d["w_up"], d["w_down"], d["gamma"], 1e-5)
    for t in (1, 2, 4, 8):
        s = sharded_mlp(d["x"], d["w_gate"], d["w_up"], d["w_down"], t, d["gamma"], 1e-5)
        assert relerr(s["sum"], ref["y"]) < 1e-12, t
        gcat = np.concatenate([r["gate"] for r in s["ranks"]], axis=1)
        acat = np.concatenate([r["a"] for r in s["ranks"]], axis=1)
        assert relerr(gcat, ref["gate"]) < 1e-12 and relerr(acat, ref["a"]) < 1e-12


def small_layer(seed=41, B=3, H=32, I=64, n_q=8, n_kv=8, d=4, cap=10):
    a = W.attention_inputs(seed, H, n_q, n_kv, d, B, cap, "f32", "random")
    m = W.mlp_inputs(seed, H, I, B, "f32", "random")
    w = {"gamma1": a["gamma"], "w_q": a["w_q"], "w_k": a["w_k"], "w_v": a["w_v"], "w_o": a["w_o"],
         "gamma2": m["gamma"], "w_gate": m["w_gate"], "w_up": m["w_up"], "w_down": m["w_down"]}
    return a["x"], w, a["k_cache"], a["v_cache"]


def pin_sharded_layer(sharded_layer, layer):
    for n_q, n_kv in [(8, 8), (16, 8), (8, 2)]:          # (8, 2) at t = 4, 8: kv heads replicated
        x, w, K, V = small_layer(n_q=n_q, n_kv=n_kv)
        for residual in (True, False):
            ref = layer(x, w, K, V, 7, n_q, n_kv, 4, 1e-5, residual)
            for t in (1, 2, 4, 8):
                s = sharded_layer(x, w, K, V, 7, n_q, n_kv, 4, t, 1e-5, residual)
                assert relerr(s["out"], ref["out"]) < 1e-12, (n_q, t, residual)
                assert relerr(s["h"], ref["h"]) < 1e-12
                ocat = np.concatenate([r["o"] for r in s["attn"]], axis=1)
                assert relerr(ocat, ref["attn"]["o"]) < 1e-12
                qcat = np.concatenate([r["q"] for r in s["attn"]], axis=1)
                assert relerr(qcat, ref["attn"]["q"]) < 1e-12


def pin_layer_literal_flow(layer, attention_block, mlp_block):
    """Without residuals the layer is mlp(attention(x)): the pseudocode's flow."""
    x, w, K, V = small_layer()
    got = layer(x, w, K, V, 7, 8, 8, 4, 1e-5, False)["out"]
    at = attention_block(x, w["w_q"], w["w_k"], w["w_v"], w["w_o"], K, V, 7, 8, 8, 4, w["gamma1"], 1e-5)
    ref = mlp_block(at["y"], w["w_gate"], w["w_up"], w["w_down"], w["gamma2"], 1e-5)["y"]
    assert np.array_equal(got, ref)


def pin_layer_vs_naive(layer):
    """The whole layer against brute-force loops, KV append included."""
    B, H, I, n_q, n_kv, d, cap, kv_len = 2, 8, 12, 4, 2, 2, 5, 4
    x, w, K, V = small_layer(seed=43, B=B, H=H, I=I, n_q=n_q, n_kv=n_kv, d=d, cap=cap)
    K0, V0 = K.copy(), V.copy()
    got = layer(x, w, K, V, kv_len, n_q, n_kv, d, 1e-5, True)
    u = naive.rmsnorm(x, w["gamma1"], 1e-5)
    q = naive.matmul(u, w["w_q"]); k = naive.matmul(u, w["w_k"]); v = naive.matmul(u, w["w_v"])
    Kn = K.astype(np.float64).copy(); Vn = V.astype(np.float64).copy()
    for b in range(B):
        for g in range(n_kv):
            Kn[b, g, kv_len - 1] = k[b][g * d:(g + 1) * d]
            Vn[b, g, kv_len - 1] = v[b][g * d:(g + 1) * d]
    o = naive.decode_attention(q, Kn, Vn, kv_len, n_q, n_kv, d)
    y = naive.matmul(o, w["w_o"])
    h = [[float(x[i][j]) + y[i][j] for j in range(H)] for i in range(B)]
    m = naive.mlp(h, w["w_gate"], w["w_up"], w["w_down"], w["gamma2"], 1e-5)
    out = [[h[i][j] + m[i][j] for j in range(H)] for i in range(B)]
    assert relerr(got["out"], out) < 1e-13
    assert relerr(got["attn"]["k_cache"], Kn) < 1e-13
    keep = [j for j in range(cap) if j != kv_len - 1]
    assert np.array_equal(got["attn"]["k_cache"][:, :, keep], Kn[:, :, keep])
    assert np.array_equal(got["attn"]["v_cache"][:, :, keep], Vn[:, :, keep])
    # the input caches are left untouched
    assert np.array_equal(K, K0) and np.array_equal(V, V0)


def small_prefill(seed=45, B=2, S=5, H=16, I=24, n_q=4, n_kv=2, d=4, cap=9):
    """A token block x [B, S, H] and the weights and caches of a small layer."""
    _, w, K, V = small_layer(seed=seed, B=B, H=H, I=I, n_q=n_q, n_kv=n_kv, d=d, cap=cap)
    x = W.storage_round(W.normal(seed, W.Q_PREFILL, (B, S, H)), "f32")
    return x, w, K, V


def pin_layer_prefill_one_token(layer_prefill, layer):
    """A block of one token per sequence is a decode step."""
    x, w, K, V = small_prefill(S=1)
    for kv_len in (1, 6, 9):
        for residual in (True, False):
            got = layer_prefill(x, w, K, V, kv_len, 4, 2, 4, 1e-5, residual)
            ref = layer(x[:, 0], w, K, V, kv_len, 4, 2, 4, 1e-5, residual)
            assert relerr(got["out"][:, 0], ref["out"]) < 1e-13, kv_len
            assert relerr(got["attn"]["k_cache"], ref["attn"]["k_cache"]) < 1e-13
            assert relerr(got["attn"]["v_cache"], ref["attn"]["v_cache"]) < 1e-13


def pin_layer_prefill_chunks(layer_prefill):
    """Prefilling a block in two chunks through the cache gives the block's result."""
    x, w, K, V = small_prefill(S=6)
    kv_len = 8
    whole = layer_prefill(x, w, K, V, kv_len, 4, 2, 4, 1e-5, True)
    for s1 in (1, 2, 5):
        first = layer_prefill(x[:, :s1], w, K, V, kv_len - 6 + s1, 4, 2, 4, 1e-5, True)
        second = layer_prefill(x[:, s1:], w, first["attn"]["k_cache"], first["attn"]["v_cache"], kv_len, 4, 2, 4,
                               1e-5, True)
        out = np.concatenate([first["out"], second["out"]], axis=1)
        assert relerr(out, whole["out"]) < 1e-13, s1
        assert relerr(second["attn"]["k_cache"], whole["attn"]["k_cache"]) < 1e-13


def pin_layer_prefill_vs_naive(layer_prefill):
    """The layer over a token block against brute-force loops, the block's KV append included."""
    B, S, H, I, n_q, n_kv, d, cap, kv_len = 2, 3, 8, 12, 4, 2, 2, 6, 5
    x, w, K, V = small_prefill(seed=47, B=B, S=S, H=H, I=I, n_q=n_q, n_kv=n_kv, d=d, cap=cap)
    K0, V0 = K.copy(), V.copy()
    got = layer_prefill(x, w, K, V, kv_len, n_q, n_kv, d, 1e-5, True)
    rows = [x[b, i] for b in range(B) for i in range(S)]            # token rows, sequence-major
    u = naive.rmsnorm(rows, w["gamma1"], 1e-5)
    q = naive.matmul(u, w["w_q"]); k = naive.matmul(u, w["w_k"]); v = naive.matmul(u, w["w_v"])
    Kn = K.astype(np.float64).copy(); Vn = V.astype(np.float64).copy()
    for b in range(B):
        for i in range(S):
            for g in range(n_kv):
                Kn[b, g, kv_len - S + i] = k[b * S + i][g * d:(g + 1) * d]
                Vn[b, g, kv_len - S + i] = v[b * S + i][g * d:(g + 1) * d]
    qb = [[q[b * S + i] for i in range(S)] for b in range(B)]
    o = naive.prefill_attention(qb, Kn, Vn, kv_len, n_q, n_kv, d)
    y = naive.matmul([o[b][i] for b in range(B) for i in range(S)], w["w_o"])
    h = [[float(rows[r][j]) + y[r][j] for j in range(H)] for r in range(B * S)]
    m = naive.mlp(h, w["w_gate"], w["w_up"], w["w_down"], w["gamma2"], 1e-5)
    out = [[h[r][j] + m[r][j] for j in range(H)] for r in range(B * S)]
    assert relerr(got["out"].reshape(B * S, H), out) < 1e-13
    assert relerr(got["attn"]["k_cache"], Kn) < 1e-13
    assert relerr(got["attn"]["v_cache"], Vn) < 1e-13
    assert np.array_equal(K, K0) and np.array_equal(V, V0)


def pin_sharded_layer_prefill(sharded_layer_prefill, layer_prefill):
    for n_q, n_kv in [(8, 8), (16, 8)]:
        x, w, K, V = small_prefill(seed=49, B=2, S=4, H=32, I=64, n_q=n_q, n_kv=n_kv, d=4, cap=10)
        for residual in (True, False):
            ref = layer_prefill(x, w, K, V, 7, n_q, n_kv, 4, 1e-5, residual)
            for t in (1, 2, 4, 8):
                s = sharded_layer_prefill(x, w, K, V, 7, n_q, n_kv, 4, t, 1e-5, residual)
                assert relerr(s["out"], ref["out"]) < 1e-12, (n_q, t, residual)
                assert relerr(s["h"], ref["h"]) < 1e-12
                for a, p in zip(s["attn"], s["plans"]):
                    kb, kn = p["kv_head_begin"], p["kv_heads"]
                    assert relerr(a["k_cache"], ref["attn"]["k_cache"][:, kb:kb + kn]) < 1e-13


def pin_moe_route(moe_route):
    """Top-k routing on hand-computed cases."""
    g = moe_route(np.array([[1.0, 3.0, 2.0, 0.0]]), 2)
    w1 = 1.0 / (1.0 + math.exp(-1.0))                # e^3 / (e^3 + e^2)
    assert np.allclose(g, [[0.0, w1, 1.0 - w1, 0.0]], rtol=0, atol=1e-15)
    g = moe_route(np.array([[5.0, 5.0, 5.0, 1.0]]), 2)  # ties go to the lower index
    assert np.allclose(g, [[0.5, 0.5, 0.0, 0.0]], rtol=0, atol=1e-15)
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((6, 8))
    one = moe_route(logits, 1)
    assert np.array_equal(one, np.eye(8)[np.argmax(logits, axis=1)])
    from scipy.special import softmax as sp_softmax
    assert np.allclose(moe_route(logits, 8), sp_softmax(logits, axis=1), rtol=0, atol=1e-14)
    g2 = moe_route(logits, 2)
    assert np.allclose(g2.sum(axis=1), 1.0, atol=1e-15) and np.all((g2 > 0).sum(axis=1) == 2)
    top2 = np.argsort(-logits, axis=1, kind="stable")[:, :2]
    assert all(set(np.nonzero(g2[t])[0]) == set(top2[t]) for t in range(6))


def small_moe(seed=61, m=5, H=16, I=12, E=4):
    x = W.storage_round(W.normal(seed, W.X, (m, H)), "f32")
    gamma = W.gamma(seed, W.GAMMA2, H, "random", "f32")
    w_router = W.storage_round(W.normal(seed, W.ATTN_IN, (H, E)), "f32")
    experts = []
    for e in range(E):
        mi = W.mlp_inputs(seed * 100 + e, H, I, 1, "f32")
        experts.append((mi["w_gate"], mi["w_up"], mi["w_down"]))
    return x, gamma, w_router, experts


def pin_moe_identical_and_single(moe_block, mlp_block):
    """Identical experts give the dense MLP (gates sum to one); so does one expert with k=1."""
    x, gamma, w_router, experts = small_moe()
    same = [experts[0]] * 4
    ref = mlp_block(x, *experts[0], gamma, 1e-5)["y"]
    for k in (1, 2, 4):
        assert relerr(moe_block(x, gamma, w_router, same, k, 1e-5)["y"], ref) < 1e-13, k
    assert relerr(moe_block(x, gamma, w_router[:, :1], experts[:1], 1, 1e-5)["y"], ref) < 1e-13


def pin_moe_vs_naive(moe_block):
    """The MoE FFN against brute-force loops: routing by hand, then each chosen expert."""
    x, gamma, w_router, experts = small_moe(seed=63, m=3, H=6, I=5, E=4)
    k = 2
    got = moe_block(x, gamma, w_router, experts, k, 1e-5)
    u = naive.rmsnorm(x, gamma, 1e-5)
    logits = naive.matmul(u, w_router)
    out = [[0.0] * 6 for _ in range(3)]
    for t in range(3):
        order = sorted(range(4), key=lambda e: (-logits[t][e], e))[:k]
        mx = max(logits[t][e] for e in order)
        den = sum(math.exp(logits[t][e] - mx) for e in order)
        for e in order:
            w = math.exp(logits[t][e] - mx) / den
            y = naive.mlp([u[t]], *experts[e])[0]
            for j in range(6):
                out[t][j] += w * y[j]
    assert relerr(got["y"], out) < 1e-13


def pin_rank_moe(rank_moe, moe_block, rank_plan, ModelDesc):
    """Every expert sharded like the dense MLP: the rank partials sum to the unsharded MoE FFN."""
    x, gamma, w_router, experts = small_moe(seed=65, m=4, H=16, I=16, E=4)
    ref = moe_block(x, gamma, w_router, experts, 2, 1e-5)
    for t in (1, 2, 4):
        desc = ModelDesc(hidden=16, intermediate=16)
        parts = [rank_moe(x, gamma, w_router, experts, ref["gates"], rank_plan(desc, t, r), 1e-5)["partial"]
                 for r in range(t)]
        assert relerr(sum(parts), ref["y"]) < 1e-12, t


def pin_kv_replication(rank_plan, ModelDesc):
    """t > n_kv: each rank holds the one kv head its q heads read; its KV cache is one head's."""
    d = ModelDesc(hidden=32, intermediate=64, n_q_heads=8, n_kv_heads=2, head_dim=4, n_layers=2, seq_len=10,
                  batch=3, bytes_per_elem=2)
    for t, heads in [(4, [0, 0, 1, 1]), (8, [0, 0, 0, 0, 1, 1, 1, 1])]:
        for r in range(t):
            p = rank_plan(d, t, r)
            assert p["kv_heads"] == 1 and p["kv_head_begin"] == heads[r], (t, r)
            group = 8 // 2
            assert all(h // group == p["kv_head_begin"]
                       for h in range(p["q_head_begin"], p["q_head_begin"] + p["q_heads"]))
            assert p["qkv_cols"] == (8 // t + 2) * 4
            assert p["kv_bytes_rank"] == 2 * 2 * 1 * 4 * 10 * 2 * 3       # 2 (k, v) x layers x 1 head x d x seq x bytes x batch

