"""GPU parity at the edges of the launch plans and at the timed full sizes.

- the decode attention stage over more than 16 sequences (the QKV projection with
  its KV-cache append runs over several 16-token blocks, then attention on the
  same batch), every rank's appended k, v and attention partial checked;
- seeded random decode-layer shapes, both stages of every rank (kv-head
  replication, odd hidden and intermediate sizes, batches across 16-token blocks);
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


# ---------------------------------------------------------------- seeded random layer shapes, decode

def _random_layer_cases(n_cases=10, seed=2026):
    """Seeded decode-layer shapes: head sizes 64 and 128, 1-8 kv heads, groups of 1-8, every t in 1..8
    the head counts allow (kv-head replication where t exceeds them), hidden and intermediate sizes off
    the tile multiples, 1-40 sequences, caches of 1-3000 keys with spare capacity."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n_cases:
        d = int(rng.choice([64, 128]))
        nkv = int(rng.choice([1, 2, 4, 8]))
        nq = nkv * int(rng.choice([1, 2, 4, 8]))
        ts = [t for t in range(1, 9) if nq % t == 0 and (nkv % t == 0 or t % nkv == 0)]
        t = int(rng.choice(ts))
        H = 8 * int(rng.integers(8, 385))
        inter = t * 8 * int(rng.integers(4, 161))
        B = int(rng.choice([1, 2, 5, 16, 17, 40]))
        kv_len = int(rng.integers(1, 3001))
        cap = kv_len + int(rng.integers(0, 65))
        cases.append((H, inter, nq, nkv, d, t, B, kv_len, cap))
    return cases


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", _random_layer_cases(), ids=lambda c: "x".join(map(str, c)))
def test_layer_decode_random_shapes(case):
    """Both stages of every rank: appended k, v, the attention partial and the MLP partial against the
    oracle's per-rank shards (the MLP stage reads x, so each stage is checked on its own)."""
    H, inter, nq, nkv, d, t, B, kv_len, cap = case
    say(f"random decode layer: hidden {H}, intermediate {inter}, {nq}/{nkv} heads, d {d}, t={t}, batch {B}, "
        f"kv_len {kv_len}, capacity {cap}")
    wid = 500 + (H + inter + kv_len) % 400
    a = W.attention_inputs(wid, H, nq, nkv, d, B, cap, "bf16", "random")
    mi = W.mlp_inputs(wid, H, inter, B, "bf16", "random")
    desc = tp.make_desc(H, inter, nq, nkv, d, n_layers=1, seq_len=cap, batch=B)
    odesc = OP.ModelDesc(hidden=H, intermediate=inter, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, seq_len=cap,
                         batch=B)
    x = dev(a["x"], "bf16")
    g1, g2 = dev(a["gamma"], "bf16"), dev(mi["gamma"], "bf16")
    for r in range(t):
        p = tp.tp_shard_plan(desc, t, r)
        op = OP.rank_plan(odesc, t, r)
        rw = rank_weights(a, mi, p, d, g1, g2)
        kb, kn = p.kv_head_begin, p.kv_heads
        kc = dev(a["k_cache"][:, kb:kb + kn], "bf16")
        vc = dev(a["v_cache"][:, kb:kb + kn], "bf16")
        pa, pm = empty((B, H), torch.float32), empty((B, H), torch.float32)
        tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_ATTN, rw, x, pa, kv={"k": kc, "v": vc, "kv_len": kv_len})
        tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, rw, x, pm)
        torch.cuda.synchronize()
        sa = S.rank_attention(a["x"], a["w_q"], a["w_k"], a["w_v"], a["w_o"], a["k_cache"], a["v_cache"], kv_len,
                              nq, nkv, d, op, a["gamma"])
        sm = S.rank_mlp(a["x"], mi["w_gate"], mi["w_up"], mi["w_down"], op, mi["gamma"])
        check(f"rank{r} appended k", host(kc)[:, :, kv_len - 1], sa["k_cache"][:, :, kv_len - 1], TOL["bf16"])
        check(f"rank{r} appended v", host(vc)[:, :, kv_len - 1], sa["v_cache"][:, :, kv_len - 1], TOL["bf16"])
        check(f"rank{r} attention partial", host(pa), sa["partial"], TOL["bf16"])
        check(f"rank{r} MLP partial", host(pm), sm["partial"], TOL["bf16"])
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


# ---------------------------------------------------------------- MoE over per-expert token lists (prefill)

def _moe_inputs(seed, H, I, E, m):
    inp = W.moe_inputs(seed, H, I, E, m, "bf16")
    return inp["x"], inp["gamma"], inp["w_router"], inp["experts"]


def _moe_rank_phys(experts, p):
    b, c = p.inter_begin, p.inter_cols
    wg = np.concatenate([phys(g[:, b:b + c]) for g, _, _ in experts], axis=0)
    wu = np.concatenate([phys(u[:, b:b + c]) for _, u, _ in experts], axis=0)
    wd = np.concatenate([phys(d[b:b + c, :]) for _, _, d in experts], axis=1)
    return wg, wu, wd


def _run_moe(x, gamma, w_router, experts, E, k, t, H, I):
    m = x.shape[0]
    desc = tp.make_desc(H, I)
    xd, gd, rd = dev(x, "bf16"), dev(gamma, "bf16"), dev(phys(w_router), "bf16")
    parts, gates, logits, plans = [], [], [], []
    for r in range(t):
        p = tp.tp_shard_plan(desc, t, r)
        wg, wu, wd = _moe_rank_phys(experts, p)
        w = {"norm": gd, "w_router": rd, "w_gate": dev(wg, "bf16"), "w_up": dev(wu, "bf16"),
             "w_down": dev(wd, "bf16")}
        part = empty((m, H), torch.float32)
        g = empty((m, E), torch.float32)
        lg = empty((m, E), torch.float32)
        tp.tp_moe_shard_forward(w, xd, part, E, k, p.inter_cols, gates=g, logits=lg)
        torch.cuda.synchronize()
        del w, wg, wu, wd
        parts.append(part); gates.append(g); logits.append(lg); plans.append(p)
    out = empty((m, H), torch.float32)
    tp.tp_partial_sum(parts, out)
    torch.cuda.synchronize()
    return parts, gates, logits, out


def _check_routing(gates, logits, k, E, t):
    lg0, g0 = host(logits[0]), host(gates[0])
    for r in range(1, t):
        assert np.array_equal(host(gates[r]), g0), "ranks disagree on the routing"
    # the routing decision taken in the kernel's precision: top-k of the GPU's logits
    g_ref = L.moe_route(lg0, k)
    assert np.array_equal(g0 > 0, g_ref > 0), "top-k selection differs"
    assert np.max(np.abs(g0 - g_ref)) < 1e-5
    return g0


GROUPED_MOE_CASES = [
    # hidden, intermediate (per expert), experts, top_k, t, tokens
    (512, 1024, 8, 2, 2, 300),       # ragged expert counts, one tile each
    (1024, 2816, 8, 2, 2, 1000),     # several expert tiles, ragged K of neither
    (256, 512, 4, 1, 1, 600),        # top-1
    (256, 512, 8, 8, 1, 130),        # every expert for every token: eight slots
    (384, 784, 16, 3, 2, 257),       # 16 experts, top-3, a token past one 256-row tile
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", GROUPED_MOE_CASES, ids=lambda c: "x".join(map(str, c)))
def test_moe_grouped_bf16(case):
    H, I, E, k, t, m = case
    x, gamma, w_router, experts = _moe_inputs(110 + E + k, H, I, E, m)
    parts, gates, logits, out = _run_moe(x, gamma, w_router, experts, E, k, t, H, I)
    ref = L.moe_block(x, gamma, w_router, experts, k)
    check("router logits", host(logits[0]), ref["logits"], TOL["bf16"])
    g0 = _check_routing(gates, logits, k, E, t)
    odesc = OP.ModelDesc(hidden=H, intermediate=I)
    small = m * H * I * E <= 2e9      # the sharded oracle's einsum products run on one thread
    for r in range(t):
        op = OP.rank_plan(odesc, t, r)
        if small:
            pr = S.rank_moe(x, gamma, w_router, experts, g0, op)["partial"]
        else:
            b, c = op["inter_begin"], op["inter_cols"]
            ex_r = [(g[:, b:b + c], u[:, b:b + c], d[b:b + c, :]) for g, u, d in experts]
            pr = L.moe_block(x, gamma, w_router, ex_r, k, gates=g0)["y"]
        check(f"rank{r} MoE partial", host(parts[r]), pr, TOL["bf16"])
    yref = L.moe_block(x, gamma, w_router, experts, k, gates=g0)["y"]
    check(f"sum of {t} MoE partials", host(out), yref, TOL["bf16"])


@pytest.mark.timeout(600)
def test_moe_grouped_idle_and_full_experts():
    """A router that sends every token to experts 0 and 1: those two run over all 600 tokens (three
    row tiles), the other six over none."""
    H, I, E, k, t, m = 256, 512, 8, 2, 2, 600
    x, gamma, w_router, experts = _moe_inputs(131, H, I, E, m)
    x = W.to_bf16(np.abs(x) + 1.0)
    w_router = W.to_bf16(np.concatenate([np.full((H, 1), 0.05), np.full((H, 1), 0.03),
                                         W.normal(131, 40, (H, E - 2), 0.001)], axis=1).astype(np.float32))
    gamma = np.ones(H, np.float32)
    parts, gates, logits, out = _run_moe(x, gamma, w_router, experts, E, k, t, H, I)
    g0 = _check_routing(gates, logits, k, E, t)
    assert np.all(g0[:, 0] > 0) and np.all(g0[:, 1] > 0) and not np.any(g0[:, 2:])
    yref = L.moe_block(x, gamma, w_router, experts, k, gates=g0)["y"]
    check("sum of 2 MoE partials", host(out), yref, TOL["bf16"])


@pytest.mark.timeout(900)
def test_moe_grouped_mixtral_prefill():
    """The Mixtral-8x7B-shaped MoE FFN shard (hidden 4096, 8 experts of intermediate 14336, top-2, t=2)
    over 4096 prefill tokens, every row: each rank's partial against the oracle's MoE block on that
    rank's column / row blocks of every expert (BLAS products, the GPU's routing), and their sum."""
    H, I, E, k, t, m = 4096, 14336, 8, 2, 2, 4096
    say("drawing the Mixtral-shaped experts")
    x, gamma, w_router, experts = _moe_inputs(9, H, I, E, m)
    parts, gates, logits, out = _run_moe(x, gamma, w_router, experts, E, k, t, H, I)
    g0 = _check_routing(gates, logits, k, E, t)
    counts = np.count_nonzero(g0, axis=0)
    say(f"  tokens per expert: {counts.tolist()}")
    odesc = OP.ModelDesc(hidden=H, intermediate=I)
    refs = []
    for r in range(t):
        op = OP.rank_plan(odesc, t, r)
        b, c = op["inter_begin"], op["inter_cols"]
        ex_r = [(L.f64(g[:, b:b + c]), L.f64(u[:, b:b + c]), L.f64(d[b:b + c, :])) for g, u, d in experts]
        say(f"oracle: rank {r}")
        yr = L.moe_block(x, gamma, w_router, ex_r, k, gates=g0)["y"]
        check(f"rank{r} MoE partial (all rows)", host(parts[r]), yr, TOL["bf16"])
        refs.append(yr)
        del ex_r
    check("sum of 2 MoE partials (all rows)", host(out), S.sum_partials(refs), TOL["bf16"])
