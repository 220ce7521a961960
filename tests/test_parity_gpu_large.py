"""GPU parity at the edges of the launch plans and at the timed full sizes.

- the decode attention stage over more than 16 sequences (the QKV projection with
  its KV-cache append runs over several 16-token blocks, then attention on the
  same batch), every rank's appended k, v and attention partial checked;
- the 70B-shaped layer prefill at t=8 over batch 2 x 2048 tokens, the timed
  prefill-layer shape, every row of the sums and of two ranks' partials;
- split-K decode projections with more row tiles than the workspace holds
  completion counters, so the tiles run in several launches.

Each compares the HIP path, called through the C ABI, with the float64 oracle,
max |err| / max |ref| <= 2e-2 (bf16) or 1e-4 (float32) per tensor.
"""
import numpy as np
import pytest
import torch

import megatron_tensor_transformer_amd as tp
import workloads as W
from gpu_helpers import TOL, check, dev, host, phys, say
from oracle import layer as L
from oracle import plan as OP
from oracle import sharded as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"


def empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="cuda")


def qkv_rank_phys(a, p, d):
    qb, qn, kb, kn = p.q_head_begin, p.q_heads, p.kv_head_begin, p.kv_heads
    return np.concatenate([phys(a["w_q"][:, qb * d:(qb + qn) * d]), phys(a["w_k"][:, kb * d:(kb + kn) * d]),
                           phys(a["w_v"][:, kb * d:(kb + kn) * d])], axis=0)


def rank_weights(a, mi, p, d, g1, g2):
    rw = {"attn_norm": g1, "w_qkv": dev(qkv_rank_phys(a, p, d), "bf16"),
          "w_o": dev(phys(a["w_o"][p.q_head_begin * d:(p.q_head_begin + p.q_heads) * d, :]), "bf16"),
          "mlp_norm": g2}
    if mi is not None:
        b, c = p.inter_begin, p.inter_cols
        rw["w_gate"] = dev(phys(mi["w_gate"][:, b:b + c]), "bf16")
        rw["w_up"] = dev(phys(mi["w_up"][:, b:b + c]), "bf16")
        rw["w_down"] = dev(phys(mi["w_down"][b:b + c, :]), "bf16")
    return rw


# ---------------------------------------------------------------- decode attention stage, batch > 16

ATTN_STAGE_CASES = [
    # hidden, q heads, kv heads, head_dim, t, sequences, kv_len, capacity, ranks checked
    (1024, 16, 4, 128, 2, 20, 300, 320, (0, 1)),
    (1024, 16, 4, 64, 2, 40, 77, 96, (0, 1)),
    (8192, 64, 8, 128, 8, 40, 1000, 1024, (0, 3, 7)),    # 70B heads at t=8
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", ATTN_STAGE_CASES, ids=lambda c: "x".join(map(str, c[:8])))
def test_decode_attention_stage_over_16_sequences(case):
    H, nq, nkv, d, t, B, kv_len, cap, ranks = case
    say(f"decode attention stage: hidden {H}, {nq}/{nkv} heads, d {d}, t={t}, batch {B}, kv_len {kv_len}")
    a = W.attention_inputs(80 + B, H, nq, nkv, d, B, cap, "bf16", "random")
    desc = tp.make_desc(H, 0, nq, nkv, d, n_layers=1, seq_len=cap, batch=B)
    odesc = OP.ModelDesc(hidden=H, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, seq_len=cap, batch=B)
    x = dev(a["x"], "bf16")
    g1 = dev(a["gamma"], "bf16")
    ref = L.attention_block(a["x"], a["w_q"], a["w_k"], a["w_v"], a["w_o"], a["k_cache"], a["v_cache"], kv_len,
                            nq, nkv, d, a["gamma"])
    for r in ranks:
        p = tp.tp_shard_plan(desc, t, r)
        rw = rank_weights(a, None, p, d, g1, None)
        kb, kn = p.kv_head_begin, p.kv_heads
        kc = dev(a["k_cache"][:, kb:kb + kn], "bf16")
        vc = dev(a["v_cache"][:, kb:kb + kn], "bf16")
        part = empty((B, H), torch.float32)
        tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_ATTN, rw, x, part, kv={"k": kc, "v": vc, "kv_len": kv_len})
        torch.cuda.synchronize()
        check(f"rank{r} appended k", host(kc)[:, :, kv_len - 1], ref["k_cache"][:, kb:kb + kn, kv_len - 1],
              TOL["bf16"])
        check(f"rank{r} appended v", host(vc)[:, :, kv_len - 1], ref["v_cache"][:, kb:kb + kn, kv_len - 1],
              TOL["bf16"])
        keep = [j for j in range(cap) if j != kv_len - 1]
        assert np.array_equal(host(kc)[:, :, keep], W.to_bf16(a["k_cache"][:, kb:kb + kn][:, :, keep]))
        sr = S.rank_attention(a["x"], a["w_q"], a["w_k"], a["w_v"], a["w_o"], a["k_cache"], a["v_cache"], kv_len,
                              nq, nkv, d, OP.rank_plan(odesc, t, r), a["gamma"])
        check(f"rank{r} attention partial", host(part), sr["partial"], TOL["bf16"])
        del rw, kc, vc


# ---------------------------------------------------------------- 70B-shaped layer prefill, t=8, 2 x 2048

@pytest.mark.timeout(900)
def test_layer_prefill_70b_t8_full_block():
    """Both stages of all 8 rank shards over batch 2 x 2048 new tokens (a prompt from scratch)."""
    H, I, nq, nkv, d, t, B, S_ = 8192, 28672, 64, 8, 128, 8, 2, 2048
    kv_len = cap = S_
    M = B * S_
    seed = 7
    say("drawing the 70B-shaped layer for a 2 x 2048-token prefill")
    a = W.attention_inputs(seed, H, nq, nkv, d, B, cap, "bf16", "random")
    mi = W.mlp_inputs(seed, H, I, 1, "bf16", "random")
    x = W.to_bf16(W.normal(seed, W.Q_PREFILL, (B, S_, H)))
    w = {"gamma1": a["gamma"], "w_q": a["w_q"], "w_k": a["w_k"], "w_v": a["w_v"], "w_o": a["w_o"],
         "gamma2": mi["gamma"], "w_gate": mi["w_gate"], "w_up": mi["w_up"], "w_down": mi["w_down"]}
    desc = tp.make_desc(H, I, nq, nkv, d, n_layers=1, seq_len=cap, batch=B)
    odesc = OP.ModelDesc(hidden=H, intermediate=I, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, seq_len=cap, batch=B)
    xd = dev(x.reshape(M, H), "bf16")
    g1, g2 = dev(a["gamma"], "bf16"), dev(mi["gamma"], "bf16")
    plans = [tp.tp_shard_plan(desc, t, r) for r in range(t)]
    rank_w, caches, attn_parts = [], [], []
    for p in plans:
        kb, kn = p.kv_head_begin, p.kv_heads
        rw = rank_weights(a, mi, p, d, g1, g2)
        kc = dev(a["k_cache"][:, kb:kb + kn], "bf16")
        vc = dev(a["v_cache"][:, kb:kb + kn], "bf16")
        part = empty((M, H), torch.float32)
        tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_ATTN, rw, xd, part,
                                  kv={"k": kc, "v": vc, "kv_len": kv_len, "new_tokens": S_})
        rank_w.append(rw)
        caches.append((kc, vc))
        attn_parts.append(part)
    h = empty((M, H), torch.bfloat16)
    tp.tp_partial_sum(attn_parts, h, residual=xd)
    mlp_parts = []
    for p, rw in zip(plans, rank_w):
        part = empty((M, H), torch.float32)
        tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, rw, h, part)
        mlp_parts.append(part)
    out = empty((M, H), torch.bfloat16)
    tp.tp_partial_sum(mlp_parts, out, residual=h)
    torch.cuda.synchronize()
    del rank_w

    say("oracle: the unsharded layer over the block")
    ref = L.layer_prefill(x, w, a["k_cache"], a["v_cache"], kv_len, nq, nkv, d)
    for r, p in enumerate(plans):
        kb, kn = p.kv_head_begin, p.kv_heads
        kc, vc = caches[r]
        check(f"rank{r} appended k block", host(kc), ref["attn"]["k_cache"][:, kb:kb + kn], TOL["bf16"])
        check(f"rank{r} appended v block", host(vc), ref["attn"]["v_cache"][:, kb:kb + kn], TOL["bf16"])
    hh = host(h)
    # two ranks' partials against the oracle's blocks on their own heads and columns (its planner's slices)
    for r in (0, 5):
        op = OP.rank_plan(odesc, t, r)
        qs = slice(op["q_head_begin"] * d, (op["q_head_begin"] + op["q_heads"]) * d)
        ks = slice(op["kv_head_begin"] * d, (op["kv_head_begin"] + op["kv_heads"]) * d)
        hs = slice(op["kv_head_begin"], op["kv_head_begin"] + op["kv_heads"])
        ar = L.attention_block_prefill(x, a["w_q"][:, qs], a["w_k"][:, ks], a["w_v"][:, ks], a["w_o"][qs, :],
                                       a["k_cache"][:, hs], a["v_cache"][:, hs], kv_len, op["q_heads"],
                                       op["kv_heads"], d, a["gamma"])
        check(f"rank{r} attention partial (all rows)", host(attn_parts[r]), ar["y"].reshape(M, H), TOL["bf16"])
        b, c = op["inter_begin"], op["inter_cols"]
        mr = L.mlp_block(hh, mi["w_gate"][:, b:b + c], mi["w_up"][:, b:b + c], mi["w_down"][b:b + c, :],
                         mi["gamma"])
        check(f"rank{r} MLP partial at the GPU's h (all rows)", host(mlp_parts[r]), mr["y"], TOL["bf16"])
    check("sum of 8 attention partials (all rows)", sum(host(q) for q in attn_parts), ref["attn"]["y"].reshape(M, H),
          TOL["bf16"])
    check("h = x + sum of 8 attention partials", hh, ref["h"].reshape(M, H), TOL["bf16"])
    mref = L.mlp_block(hh, w["w_gate"], w["w_up"], w["w_down"], w["gamma2"])
    check("sum of 8 MLP partials at the GPU's h (all rows)", sum(host(q) for q in mlp_parts), mref["y"], TOL["bf16"])
    check("layer output", host(out), ref["out"].reshape(M, H), TOL["bf16"])


# ---------------------------------------------------------------- split K with more row tiles than counters

SPLIT_TILE_CASES = [
    # m, k, n, dtype, mode: n / 8 row tiles exceed the 8192 completion counters of the workspace header
    (1, 4608, 70000, "bf16", "col"),
    (1, 4608, 70000, "bf16", "row"),
    (4, 4096, 70000, "f32", "col"),
    (1, 4608, 140000, "bf16", "swiglu"),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", SPLIT_TILE_CASES, ids=lambda c: "x".join(map(str, c)))
def test_split_k_more_tiles_than_counters(case):
    m, k, n, dt, mode = case
    seed = 300 + m
    x = W.storage_round(W.normal(seed, 0, (m, k)), dt)
    wp = W.storage_round(W.normal(seed, 1, (n, k), 0.05), dt)     # physical [n, k]
    wu = W.storage_round(W.normal(seed, 2, (n, k), 0.05), dt) if mode == "swiglu" else None
    tx, tw = dev(x, dt), dev(wp, dt)
    if mode == "row":
        y = empty((m, n), torch.float32)
        ws = torch.zeros(tp.tp_linear_workspace_bytes(m, k, n, tp.TP_BF16 if dt == "bf16" else tp.TP_F32),
                         dtype=torch.uint8, device="cuda")
        tp.tp_row_linear_partial(tx, tw, y, ws=ws)
        tp.tp_row_linear_partial(tx, tw, y, ws=ws)      # a second call finds the counters zero again
    else:
        y = empty((m, n), torch.bfloat16 if dt == "bf16" else torch.float32)
        twu = dev(wu, dt) if wu is not None else None
        tp.tp_column_linear(tx, tw, y, w_up=twu)
    torch.cuda.synchronize()
    ref = L.linear(x, wp.T)
    if mode == "swiglu":
        ref = L.swiglu(ref, L.linear(x, wu.T))
    check(f"{mode} m={m} k={k} n={n} {dt}", host(y), ref, TOL[dt])
