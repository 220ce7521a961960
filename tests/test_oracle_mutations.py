"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Each case patches one oracle function with a plausible slip (a dropped term, a
wrong sign or index, a transposed operand) and runs the pins that cover it.
"""
import numpy as np
import pytest

import oracle_pins as P
from oracle import layer as L
from oracle import plan
from oracle import sharded as S


def _all_layer_pins():
    P.pin_silu(L.silu)
    P.pin_rmsnorm(L.rmsnorm)
    P.pin_mlp_vs_naive(L.mlp_block)
    P.pin_attention_vs_naive(L.decode_attention)
    P.pin_attention_special_cases(L.decode_attention)
    P.pin_sharded_mlp(S.sharded_mlp, L.mlp_block)
    P.pin_sharded_layer(S.sharded_layer, L.layer)
    P.pin_layer_vs_naive(L.layer)


def _all_prefill_pins():
    P.pin_prefill_attention(L.prefill_attention, L.decode_attention)
    P.pin_rank_prefill(S.rank_prefill_attention, L.prefill_attention, plan.rank_plan, plan.ModelDesc)


def _all_layer_prefill_pins():
    P.pin_layer_prefill_one_token(L.layer_prefill, L.layer)
    P.pin_layer_prefill_chunks(L.layer_prefill)
    P.pin_layer_prefill_vs_naive(L.layer_prefill)
    P.pin_sharded_layer_prefill(S.sharded_layer_prefill, L.layer_prefill)


def _all_moe_pins():
    P.pin_moe_route(L.moe_route)
    P.pin_moe_identical_and_single(L.moe_block, L.mlp_block)
    P.pin_moe_vs_naive(L.moe_block)
    P.pin_rank_moe(S.rank_moe, L.moe_block, plan.rank_plan, plan.ModelDesc)


def _all_sharded_pins():
    P.pin_silu(S._silu)
    P.pin_rmsnorm(lambda x, g, eps: S._norm(x, g, eps))
    P.pin_column_concat_naive(S.column_shard, plan.rank_plan, plan.ModelDesc)
    P.pin_row_partials_sum(S.row_shard, S.sum_partials, plan.rank_plan, plan.ModelDesc)
    P.pin_sharded_mlp(S.sharded_mlp, L.mlp_block)
    P.pin_sharded_layer(S.sharded_layer, L.layer)


def _all_proj_pins():
    P.pin_attn_proj_block(L.attn_proj_block)


def _all_plan_pins():
    P.pin_kv_worked_example(plan.kv_elements_per_sequence, plan.kv_bytes_per_gpu)
    P.pin_weight_footprint(plan.weight_bytes_per_gpu)
    P.pin_head_blocks(plan.rank_plan, plan.ModelDesc)
    P.pin_workload_shapes(plan.rank_plan, plan.ModelDesc)
    P.pin_plan_errors(plan.rank_plan, plan.ModelDesc, plan.PlanError)
    P.pin_layer_weight_elements(plan.layer_weight_elements, plan.rank_plan, plan.ModelDesc)


_orig_rank_plan = plan.rank_plan
_orig_attention = L.decode_attention
_orig_rank_attention = S.rank_attention
_orig_prefill = L.prefill_attention
_orig_rank_prefill = S.rank_prefill_attention


def _prefill_strict_mask(q, k, v, kv_len, n_q, n_kv, d):
    # each token attends to positions before it but not itself (first row undefined -> use key 0 only)
    q = np.asarray(q, np.float64)
    B, S = q.shape[:2]
    out = np.zeros((B, S, n_q * d))
    for i in range(S):
        seen = max(kv_len - S + i, 1)
        out[:, i] = _orig_attention(q[:, i], k, v, seen, n_q, n_kv, d)
    return out


def _prefill_no_mask(q, k, v, kv_len, n_q, n_kv, d):
    q = np.asarray(q, np.float64)
    B, S = q.shape[:2]
    return np.stack([_orig_attention(q[:, i], k, v, kv_len, n_q, n_kv, d) for i in range(S)], axis=1)


def _prefill_positions_from_zero(q, k, v, kv_len, n_q, n_kv, d):
    # treats the block as starting at position 0 even when kv_len > S
    return _orig_prefill(q, k, v, np.shape(q)[1], n_q, n_kv, d)


def _rank_prefill_global_kv(q, k, v, kv_len, n_q, n_kv, d, p):
    # uses the global kv head index into the rank's local kv slice
    p2 = dict(p)
    p2["kv_head_begin"] = 0
    return _orig_rank_prefill(q, k, v, kv_len, n_q, n_kv, d, p2) if p["kv_head_begin"] == 0 else \
        _orig_rank_prefill(q, np.roll(k, 1, axis=1), np.roll(v, 1, axis=1), kv_len, n_q, n_kv, d, p)


_orig_append_block = L.append_kv_block
_orig_rank_attention_prefill = S.rank_attention_prefill


def _append_block_shifted(kc, vc, kn, vn, kv_len, n_kv, d):
    # writes the block one position early (starting at kv_len - S - 1)
    S_ = np.shape(kn)[1]
    if kv_len - S_ - 1 < 0:
        return _orig_append_block(kc, vc, kn, vn, kv_len, n_kv, d)
    return _orig_append_block(kc, vc, kn, vn, kv_len - 1, n_kv, d)


def _append_block_skipped(kc, vc, kn, vn, kv_len, n_kv, d):
    # attends over the cache as it was, without the block's own keys and values
    return np.asarray(kc, np.float64).copy(), np.asarray(vc, np.float64).copy()


def _append_block_token_major(kc, vc, kn, vn, kv_len, n_kv, d):
    # reads the block's k as [n_kv, S] instead of [S, n_kv] per sequence
    B, S_ = np.shape(kn)[0], np.shape(kn)[1]
    kc2 = np.asarray(kc, np.float64).copy()
    vc2 = np.asarray(vc, np.float64).copy()
    kc2[:, :, kv_len - S_:kv_len, :] = np.asarray(kn, np.float64).reshape(B, n_kv, S_, d)
    vc2[:, :, kv_len - S_:kv_len, :] = np.asarray(vn, np.float64).reshape(B, n_kv, S_, d)
    return kc2, vc2


def _rank_attention_prefill_no_norm(x, w_q, w_k, w_v, w_o, kc, vc, kv_len, n_q, n_kv, d, p, gamma=None, eps=1e-5):
    return _orig_rank_attention_prefill(x, w_q, w_k, w_v, w_o, kc, vc, kv_len, n_q, n_kv, d, p, None, eps)


def _attn_proj_x_to_wo(x, attn_in, w_q, w_k, w_v, w_o):
    # feeds the layer input to W_o instead of the attention output
    return {"q": L.linear(x, w_q), "k": L.linear(x, w_k), "v": L.linear(x, w_v), "y": L.linear(x, w_o)}


def _attn_proj_kv_swapped(x, attn_in, w_q, w_k, w_v, w_o):
    return {"q": L.linear(x, w_q), "k": L.linear(x, w_v), "v": L.linear(x, w_k), "y": L.linear(attn_in, w_o)}


def _layer_weights_one_kv(desc):
    # counts the kv heads once (K only) in the QKV weights
    H, d = desc.hidden, desc.head_dim
    return H * (desc.n_q_heads + desc.n_kv_heads) * d + desc.n_q_heads * d * H + 3 * H * desc.intermediate


_orig_moe_route = L.moe_route
_orig_rank_moe = S.rank_moe


def _moe_route_no_renorm(logits, k):
    # keeps the full-softmax probabilities of the top k instead of renormalising them
    g = _orig_moe_route(logits, k)
    full = L.softmax(np.asarray(logits, np.float64))
    return np.where(g > 0, full, 0.0)


def _moe_route_smallest(logits, k):
    return _orig_moe_route(-np.asarray(logits, np.float64), k)


def _moe_route_ties_high(logits, k):
    lg = np.asarray(logits, np.float64)
    return _orig_moe_route(lg[:, ::-1], k)[:, ::-1]


def _rank_moe_no_gates(x, gamma, w_router, experts, gates, p, eps=1e-5):
    return _orig_rank_moe(x, gamma, w_router, experts, (np.asarray(gates) > 0).astype(float), p, eps)


def _plan_replicate_round_robin(desc, t, rank):
    # t > n_kv: assigns kv heads to ranks round robin instead of by q-head group
    p = dict(_orig_rank_plan(desc, t, rank))
    if desc.n_q_heads and desc.n_kv_heads % t:
        p["kv_head_begin"] = rank % desc.n_kv_heads
    return p


def _plan_shift_heads(desc, t, rank):
    p = dict(_orig_rank_plan(desc, t, rank))
    p["q_head_begin"] = rank * p["q_heads"] + (1 if rank and p["q_heads"] > 1 else 0)
    return p


def _plan_wrong_inter(desc, t, rank):
    p = dict(_orig_rank_plan(desc, t, rank))
    p["inter_begin"] = (t - 1 - rank) * p["inter_cols"] if rank == 0 else p["inter_begin"]
    return p


def _attention_group_modulo(q, k, v, kv_len, n_q, n_kv, d):
    # query head h reads kv head h % n_kv instead of h // (n_q / n_kv)
    qq = np.asarray(q, np.float64).reshape(q.shape[0], n_q, d)
    B = qq.shape[0]
    out = np.zeros((B, n_q, d))
    for b in range(B):
        for h in range(n_q):
            g = h % n_kv
            p = L.softmax(np.asarray(k[b, g, :kv_len], np.float64) @ qq[b, h] / np.sqrt(d))
            out[b, h] = p @ np.asarray(v[b, g, :kv_len], np.float64)
    return out.reshape(B, n_q * d)


def _attention_no_scale(q, k, v, kv_len, n_q, n_kv, d):
    return _orig_attention(np.asarray(q, np.float64) * np.sqrt(d), k, v, kv_len, n_q, n_kv, d)


def _attention_short(q, k, v, kv_len, n_q, n_kv, d):
    return _orig_attention(q, k, v, max(kv_len - 1, 1), n_q, n_kv, d)


def _append_wrong_slot(kc, vc, kn, vn, kv_len, n_kv, d):
    # writes the new token at position kv_len instead of kv_len - 1
    kc2 = np.asarray(kc, np.float64).copy()
    vc2 = np.asarray(vc, np.float64).copy()
    j = min(kv_len, kc2.shape[2] - 1)
    B = kc2.shape[0]
    kc2[:, :, j] = np.asarray(kn, np.float64).reshape(B, n_kv, d)
    vc2[:, :, j] = np.asarray(vn, np.float64).reshape(B, n_kv, d)
    return kc2, vc2


def _rank_mlp_silu_on_up(x, w_gate, w_up, w_down, p, gamma=None, eps=1e-5):
    b, c = p["inter_begin"], p["inter_cols"]
    u = S._norm(x, gamma, eps)
    g = S._mm(u, S.column_shard(w_gate, b, c))
    v = S._mm(u, S.column_shard(w_up, b, c))
    a = S._silu(v) * g
    return {"gate": g, "up": v, "a": a, "partial": S._mm(a, S.row_shard(w_down, b, c))}


def _layer_mlp_reads_x(x, w, k_cache, v_cache, kv_len, n_q, n_kv, d, eps=1e-5, residual=True):
    attn = L.attention_block(x, w["w_q"], w["w_k"], w["w_v"], w["w_o"], k_cache, v_cache, kv_len,
                             n_q, n_kv, d, w.get("gamma1"), eps)
    h = L.f64(x) + attn["y"] if residual else attn["y"]
    mlp = L.mlp_block(x if residual else h, w["w_gate"], w["w_up"], w["w_down"], w.get("gamma2"), eps)
    out = h + mlp["y"] if residual else mlp["y"]
    return {"attn": attn, "h": h, "mlp": mlp, "out": out}


def _layer_out_skips_attention(x, w, k_cache, v_cache, kv_len, n_q, n_kv, d, eps=1e-5, residual=True):
    r = _orig_layer(x, w, k_cache, v_cache, kv_len, n_q, n_kv, d, eps, residual)
    if residual:
        r["out"] = L.f64(x) + r["mlp"]["y"]
    return r


def _moe_block_experts_reversed(x, gamma, w_router, experts, k, eps=1e-5, gates=None):
    u = L.rmsnorm(x, gamma, eps) if gamma is not None else L.f64(x)
    logits = L.linear(u, w_router)
    if gates is None:
        gates = L.moe_route(logits, k)
    y = np.zeros((u.shape[0], np.shape(experts[0][2])[1]))
    E = len(experts)
    for e, (wg, wu, wd) in enumerate(experts):
        y += gates[:, E - 1 - e:E - e] * L.linear(L.swiglu(L.linear(u, wg), L.linear(u, wu)), wd)
    return {"u": u, "logits": logits, "gates": gates, "y": y}


def _rank_attention_q_from_kv_block(x, w_q, w_k, w_v, w_o, k_cache, v_cache, kv_len, n_q, n_kv, d, p, gamma=None,
                                    eps=1e-5):
    # the rank reads the next rank's q heads (an off-by-one-rank slip; t = 1 has no other rank)
    p2 = dict(p)
    p2["q_head_begin"] = (p["q_head_begin"] + p["q_heads"]) % n_q
    return _orig_rank_attention(x, w_q, w_k, w_v, w_o, k_cache, v_cache, kv_len, n_q, n_kv, d, p2, gamma, eps)


_orig_layer = L.layer


MUTATIONS = {
    # elementwise
    "silu_sign": (L, "silu", lambda z: np.asarray(z, float) * L.sigmoid(-np.asarray(z, float)), _all_layer_pins),
    "silu_is_sigmoid": (L, "silu", lambda z: L.sigmoid(z), _all_layer_pins),
    "sharded_silu_half": (S, "_silu", lambda z: np.asarray(z, float) * (1 + np.tanh(0.5 * np.asarray(z, float))),
                          _all_sharded_pins),
    "rmsnorm_sum_not_mean": (L, "rmsnorm", lambda x, g, e: np.asarray(x, float) / np.sqrt(
        np.sum(np.asarray(x, float) ** 2, axis=-1, keepdims=True) + e) * np.asarray(g, float), _all_layer_pins),
    "rmsnorm_axis0": (L, "rmsnorm", lambda x, g, e: np.asarray(x, float) / np.sqrt(
        np.mean(np.asarray(x, float) ** 2, axis=0, keepdims=True) + e) * np.asarray(g, float), _all_layer_pins),
    "rmsnorm_eps_outside": (L, "rmsnorm", lambda x, g, e: np.asarray(x, float) / (np.sqrt(
        np.mean(np.asarray(x, float) ** 2, axis=-1, keepdims=True)) + e) * np.asarray(g, float), _all_layer_pins),
    "rmsnorm_no_gamma": (L, "rmsnorm", lambda x, g, e: np.asarray(x, float) / np.sqrt(
        np.mean(np.asarray(x, float) ** 2, axis=-1, keepdims=True) + e), _all_layer_pins),
    "sharded_norm_no_eps": (S, "_norm", lambda x, g, e: S._f(x) / np.sqrt(
        np.mean(S._f(x) ** 2, axis=1, keepdims=True)) * (1.0 if g is None else S._f(g)), _all_sharded_pins),
    # blocks
    "swiglu_on_up": (L, "swiglu", lambda g, u: L.silu(u) * np.asarray(g, float), _all_layer_pins),
    "linear_reads_out_in": (L, "linear", lambda x, w: np.asarray(x, float) @ np.asarray(w, float).reshape(
        np.shape(w)[1], np.shape(w)[0]).T, _all_layer_pins),
    "attention_group_modulo": (L, "decode_attention", _attention_group_modulo, _all_layer_pins),
    "attention_no_scale": (L, "decode_attention", _attention_no_scale, _all_layer_pins),
    "attention_drops_last_key": (L, "decode_attention", _attention_short, _all_layer_pins),
    "append_wrong_slot": (L, "append_kv", _append_wrong_slot, _all_layer_pins),
    "prefill_strict_mask": (L, "prefill_attention", _prefill_strict_mask, _all_prefill_pins),
    "prefill_no_mask": (L, "prefill_attention", _prefill_no_mask, _all_prefill_pins),
    "prefill_positions_from_zero": (L, "prefill_attention", _prefill_positions_from_zero, _all_prefill_pins),
    "rank_prefill_wrong_kv_head": (S, "rank_prefill_attention", _rank_prefill_global_kv, _all_prefill_pins),
    "prefill_block_append_shifted": (L, "append_kv_block", _append_block_shifted, _all_layer_prefill_pins),
    "prefill_block_append_skipped": (L, "append_kv_block", _append_block_skipped, _all_layer_prefill_pins),
    "prefill_block_append_transposed": (L, "append_kv_block", _append_block_token_major, _all_layer_prefill_pins),
    "rank_attention_prefill_no_norm": (S, "rank_attention_prefill", _rank_attention_prefill_no_norm,
                                       _all_layer_prefill_pins),
    "moe_route_not_renormalised": (L, "moe_route", _moe_route_no_renorm, _all_moe_pins),
    "moe_route_picks_smallest": (L, "moe_route", _moe_route_smallest, _all_moe_pins),
    "moe_route_ties_to_higher_index": (L, "moe_route", _moe_route_ties_high, _all_moe_pins),
    "rank_moe_ignores_gate_weights": (S, "rank_moe", _rank_moe_no_gates, _all_moe_pins),
    "attn_proj_feeds_x_to_w_o": (L, "attn_proj_block", _attn_proj_x_to_wo, _all_proj_pins),
    "attn_proj_swaps_k_and_v": (L, "attn_proj_block", _attn_proj_kv_swapped, _all_proj_pins),
    "layer_mlp_reads_x_not_h": (L, "layer", _layer_mlp_reads_x, _all_layer_pins),
    "layer_out_skips_attention": (L, "layer", _layer_out_skips_attention, _all_layer_pins),
    "moe_gates_of_reversed_experts": (L, "moe_block", _moe_block_experts_reversed, _all_moe_pins),
    # decomposition
    "rank_mlp_silu_on_up": (S, "rank_mlp", _rank_mlp_silu_on_up, _all_sharded_pins),
    "rank_attention_wrong_q_heads": (S, "rank_attention", _rank_attention_q_from_kv_block, _all_sharded_pins),
    "sum_drops_last_rank": (S, "sum_partials", lambda parts, residual=None: np.sum(
        [np.asarray(p, float) for p in parts[:-1]] or [np.zeros_like(parts[0])], axis=0)
        + (0.0 if residual is None else np.asarray(residual, float)), _all_sharded_pins),
    "column_shard_off_by_one": (S, "column_shard", lambda w, b, c: np.asarray(w)[:, b + (1 if b else 0):b + c + (1 if b else 0)],
                                _all_sharded_pins),
    "row_shard_as_columns": (S, "row_shard", lambda w, b, c: np.asarray(w)[b:b + c, :][:, ::-1], _all_sharded_pins),
    "rank_attention_residual_per_rank": (S, "sum_partials", lambda parts, residual=None: np.sum(
        [np.asarray(p, float) + (0.0 if residual is None else np.asarray(residual, float)) for p in parts], axis=0),
        _all_sharded_pins),
    # planner
    "kv_missing_factor_two": (plan, "kv_elements_per_sequence", lambda L_, h, d, s: L_ * h * d * s, _all_plan_pins),
    "kv_not_divided_by_t": (plan, "kv_bytes_per_gpu", lambda L_, h, d, s, b, B, t:
                            plan.kv_elements_per_sequence(L_, h, d, s) * b * B, _all_plan_pins),
    "weights_not_divided": (plan, "weight_bytes_per_gpu", lambda total, t: total, _all_plan_pins),
    "heads_shifted": (plan, "rank_plan", _plan_shift_heads, _all_plan_pins),
    "layer_weights_count_kv_once": (plan, "layer_weight_elements", _layer_weights_one_kv, _all_plan_pins),
    "inter_block_swapped": (plan, "rank_plan", _plan_wrong_inter, _all_sharded_pins),
    "kv_replicated_round_robin": (plan, "rank_plan", _plan_replicate_round_robin, _all_sharded_pins),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    mod, attr, fn, pins = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    if mod is plan:
        # the sharded module reaches the planner through its own import of the module
        monkeypatch.setattr(S._plan, attr, fn)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        pins()
