"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Every workload is drawn by ``workloads`` (seeded, storage-rounded), sliced per
rank on the GPU side with the library's own planner, run rank by rank on the
one device, summed on device, and compared with the float64 oracle: max |err|
/ max |ref| <= 1e-4 for float32 workloads and <= 2e-2 for bf16 workloads.
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
    say(f"device: {torch.cuda.get_device_name(0)}")


def empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="cuda")


def mlp_rank_phys(inp, p):
    b, c = p.inter_begin, p.inter_cols
    return phys(inp["w_gate"][:, b:b + c]), phys(inp["w_up"][:, b:b + c]), phys(inp["w_down"][b:b + c, :])


# ---------------------------------------------------------------- tiny MLP, float32, t=2

def test_tiny_mlp_f32():
    wl = W.WORKLOADS[1]
    m, H, I, t = wl.tokens[0], wl.hidden, wl.intermediate, wl.t
    inp = W.mlp_inputs(1, H, I, m, "f32")
    ref = L.mlp_block(inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"])
    sref = S.sharded_mlp(inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"], t)
    desc = tp.make_desc(H, I, bytes_per_elem=4)
    x = dev(inp["x"], "f32")
    parts, parts_fused = [], []
    for r in range(t):
        p = tp.tp_shard_plan(desc, t, r)
        wg, wu, wd = [dev(a, "f32") for a in mlp_rank_phys(inp, p)]
        c = p.inter_cols
        g, u, a, a2 = (empty((m, c), torch.float32) for _ in range(4))
        tp.tp_column_linear(x, wg, g)
        tp.tp_column_linear(x, wu, u)
        tp.tp_swiglu(g, u, a)
        tp.tp_column_linear(x, wg, a2, w_up=wu)
        pr, pr2 = empty((m, H), torch.float32), empty((m, H), torch.float32)
        tp.tp_row_linear_partial(a, wd, pr)
        tp.tp_row_linear_partial(a2, wd, pr2)
        torch.cuda.synchronize()
        rr = sref["ranks"][r]
        check(f"rank{r} gate", host(g), rr["gate"], TOL["f32"])
        check(f"rank{r} up", host(u), rr["up"], TOL["f32"])
        check(f"rank{r} swiglu", host(a), rr["a"], TOL["f32"])
        check(f"rank{r} fused swiglu", host(a2), rr["a"], TOL["f32"])
        check(f"rank{r} partial", host(pr), rr["partial"], TOL["f32"])
        parts.append(pr)
        parts_fused.append(pr2)
    out, out2 = empty((m, H), torch.float32), empty((m, H), torch.float32)
    tp.tp_partial_sum(parts, out)
    tp.tp_partial_sum(parts_fused, out2)
    torch.cuda.synchronize()
    check("sum of partials", host(out), ref["y"], TOL["f32"])
    check("sum of partials (fused)", host(out2), ref["y"], TOL["f32"])


# ---------------------------------------------------------------- Llama-3-8B-shaped MLP decode, bf16, t=4

@pytest.fixture(scope="module")
def mlp8b():
    wl = W.WORKLOADS[2]
    inp = W.mlp_inputs(2, wl.hidden, wl.intermediate, 16, "bf16", "random")
    desc = tp.make_desc(wl.hidden, wl.intermediate)
    ranks = []
    for r in range(wl.t):
        p = tp.tp_shard_plan(desc, wl.t, r)
        ranks.append((p, [dev(a, "bf16") for a in mlp_rank_phys(inp, p)]))
    return wl, inp, desc, ranks


@pytest.mark.parametrize("gamma_mode", ["ones", "random"])
@pytest.mark.parametrize("m", [1, 4, 16])
def test_mlp_decode_bf16(mlp8b, m, gamma_mode):
    wl, inp, desc, ranks = mlp8b
    say(f"Llama-3-8B-shaped MLP decode shard m={m} gamma={gamma_mode}")
    gamma = np.ones(wl.hidden, np.float32) if gamma_mode == "ones" else inp["gamma"]
    xs = inp["x"][:m]                      # the batches are prefixes of one draw
    ref = L.mlp_block(xs, inp["w_gate"], inp["w_up"], inp["w_down"], gamma, wl.eps)
    sref = S.sharded_mlp(xs, inp["w_gate"], inp["w_up"], inp["w_down"], wl.t, gamma, wl.eps)
    x = dev(xs, "bf16")
    gam = dev(gamma, "bf16")
    parts = []
    for r, (p, (wg, wu, wd)) in enumerate(ranks):
        part = empty((m, wl.hidden), torch.float32)
        tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, {"mlp_norm": gam, "w_gate": wg, "w_up": wu,
                                                              "w_down": wd}, x, part)
        a = empty((m, p.inter_cols), torch.bfloat16)
        tp.tp_column_linear(x, wg, a, w_up=wu, gamma=gam, eps=wl.eps)
        torch.cuda.synchronize()
        check(f"rank{r} swiglu(norm(x))", host(a), sref["ranks"][r]["a"], TOL["bf16"])
        check(f"rank{r} partial", host(part), sref["ranks"][r]["partial"], TOL["bf16"])
        parts.append(part)
    out = empty((m, wl.hidden), torch.float32)
    tp.tp_partial_sum(parts, out)
    torch.cuda.synchronize()
    check("sum of 4 partials", host(out), ref["y"], TOL["bf16"])


@pytest.mark.parametrize("m", [1, 4, 16])
def test_mlp_decode_bf16_partials(mlp8b, m):
    """The MLP decode step with bf16 row partials and their float32 sum."""
    wl, inp, desc, ranks = mlp8b
    xs = inp["x"][:m]
    ref = L.mlp_block(xs, inp["w_gate"], inp["w_up"], inp["w_down"], inp["gamma"], wl.eps)
    sref = S.sharded_mlp(xs, inp["w_gate"], inp["w_up"], inp["w_down"], wl.t, inp["gamma"], wl.eps)
    x = dev(xs, "bf16")
    gam = dev(inp["gamma"], "bf16")
    parts = []
    for r, (p, (wg, wu, wd)) in enumerate(ranks):
        a = empty((m, p.inter_cols), torch.bfloat16)
        tp.tp_column_linear(x, wg, a, w_up=wu, gamma=gam, eps=wl.eps)
        part = empty((m, wl.hidden), torch.bfloat16)
        tp.tp_row_linear_partial_bf16(a, wd, part)
        parts.append(part)
    out = empty((m, wl.hidden), torch.bfloat16)
    tp.tp_partial_sum_bf16(parts, out)
    torch.cuda.synchronize()
    for r in range(wl.t):
        check(f"rank{r} bf16 partial", host(parts[r]), sref["ranks"][r]["partial"], TOL["bf16"])
    check("sum of 4 bf16 partials", host(out), ref["y"], TOL["bf16"])


# ---------------------------------------------------------------- 70B-shaped attention projections, t=4

def qkv_rank_phys(a, p, d):
    qb, qn, kb, kn = p.q_head_begin, p.q_heads, p.kv_head_begin, p.kv_heads
    return np.concatenate([phys(a["w_q"][:, qb * d:(qb + qn) * d]), phys(a["w_k"][:, kb * d:(kb + kn) * d]),
                           phys(a["w_v"][:, kb * d:(kb + kn) * d])], axis=0)


def test_attn_projections_bf16():
    wl = W.WORKLOADS[3]
    H, nq, nkv, d, t, m = wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t, wl.tokens[0]
    a = W.attention_inputs(3, H, nq, nkv, d, m, 1, "bf16", with_cache=False)
    attn_in = W.attn_proj_input(3, m, nq * d, "bf16")
    ref = L.attn_proj_block(a["x"], attn_in, a["w_q"], a["w_k"], a["w_v"], a["w_o"])
    desc = tp.make_desc(H, 0, nq, nkv, d)
    x = dev(a["x"], "bf16")
    qs, ks, vs, parts = [], [], [], []
    for r in range(t):
        p = tp.tp_shard_plan(desc, t, r)
        assert (p.qkv_cols, p.o_rows) == (2560, 2048)
        wqkv = dev(qkv_rank_phys(a, p, d), "bf16")
        y = empty((m, p.qkv_cols), torch.bfloat16)
        tp.tp_column_linear(x, wqkv, y)
        wo = dev(phys(a["w_o"][p.q_head_begin * d:(p.q_head_begin + p.q_heads) * d, :]), "bf16")
        ar = dev(attn_in[:, p.q_head_begin * d:(p.q_head_begin + p.q_heads) * d], "bf16")
        part = empty((m, H), torch.float32)
        tp.tp_row_linear_partial(ar, wo, part)
        torch.cuda.synchronize()
        yh = host(y)
        qs.append(yh[:, :p.o_rows])
        ks.append(yh[:, p.o_rows:p.o_rows + p.kv_heads * d])
        vs.append(yh[:, p.o_rows + p.kv_heads * d:])
        parts.append(part)
    check("Q (concat of 4 column shards)", np.concatenate(qs, 1), ref["q"], TOL["bf16"])
    check("K (concat)", np.concatenate(ks, 1), ref["k"], TOL["bf16"])
    check("V (concat)", np.concatenate(vs, 1), ref["v"], TOL["bf16"])
    out = empty((m, H), torch.float32)
    tp.tp_partial_sum(parts, out)
    torch.cuda.synchronize()
    check("W_o: sum of 4 row partials", host(out), ref["y"], TOL["bf16"])


# ---------------------------------------------------------------- 70B-shaped MLP prefill, t=4, 4096 tokens

def mlp_rows_f64(x, wg, wu, wd, chunk=1024):
    """The MLP block of the oracle (float64, BLAS products) over row chunks of x."""
    return np.concatenate([L.mlp_block(x[i:i + chunk], wg, wu, wd)["y"] for i in range(0, x.shape[0], chunk)])


@pytest.mark.timeout(900)
def test_mlp_prefill_bf16():
    """Every row of every rank's partial and of their sum, at the full 70B-shaped prefill size."""
    wl = W.WORKLOADS[4]
    H, I, t, M = wl.hidden, wl.intermediate, wl.t, wl.tokens[0]
    say("drawing the 70B-shaped MLP weights")
    inp = W.mlp_inputs(4, H, I, M, "bf16")
    desc = tp.make_desc(H, I)
    odesc = OP.ModelDesc(hidden=H, intermediate=I)
    x = dev(inp["x"], "bf16")
    rows = np.unique(np.concatenate([[0, 1, 2047, 2048, M - 1], np.random.default_rng(4).choice(M, 27, False)]))
    parts, refs = [], []
    for r in range(t):
        p = tp.tp_shard_plan(desc, t, r)
        wg, wu, wd = [dev(a, "bf16") for a in mlp_rank_phys(inp, p)]
        part = empty((M, H), torch.float32)
        tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, {"w_gate": wg, "w_up": wu, "w_down": wd}, x, part)
        torch.cuda.synchronize()
        del wg, wu, wd
        # the rank's partial is the MLP block of its own column / row blocks (the oracle's planner slices)
        op = OP.rank_plan(odesc, t, r)
        b, c = op["inter_begin"], op["inter_cols"]
        say(f"oracle: rank {r} over all {M} rows")
        ref_r = mlp_rows_f64(inp["x"], L.f64(inp["w_gate"][:, b:b + c]), L.f64(inp["w_up"][:, b:b + c]),
                             L.f64(inp["w_down"][b:b + c, :]))
        check(f"rank{r} partial (all rows)", host(part), ref_r, TOL["bf16"])
        if r == 0:
            rr = S.rank_mlp(inp["x"][rows], inp["w_gate"], inp["w_up"], inp["w_down"], op)
            check("rank0 partial (sampled rows, sharded oracle)", host(part)[rows], rr["partial"], TOL["bf16"])
        parts.append(part)
        refs.append(ref_r)
    out = empty((M, H), torch.float32)
    tp.tp_partial_sum(parts, out)
    torch.cuda.synchronize()
    # the rank-order float64 sum of the rank blocks equals the unsharded block (pinned on the oracle)
    check("sum of 4 partials (all rows)", host(out), S.sum_partials(refs), TOL["bf16"])
    ref = L.mlp_block(inp["x"][rows], inp["w_gate"], inp["w_up"], inp["w_down"])
    check("sum of 4 partials (sampled rows, unsharded)", host(out)[rows], ref["y"], TOL["bf16"])


# ---------------------------------------------------------------- 70B-shaped full layer decode, t=8

@pytest.mark.timeout(600)
def test_full_layer_decode_bf16():
    wl = W.WORKLOADS[5]
    H, I, nq, nkv, d, t, B, S_ = wl.hidden, wl.intermediate, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t, \
        wl.tokens[0], wl.kv_len
    say("drawing the 70B-shaped layer and its KV cache")
    a = W.attention_inputs(5, H, nq, nkv, d, B, S_, "bf16", "random")
    mi = W.mlp_inputs(5, H, I, B, "bf16", "random")
    w = {"gamma1": a["gamma"], "w_q": a["w_q"], "w_k": a["w_k"], "w_v": a["w_v"], "w_o": a["w_o"],
         "gamma2": mi["gamma"], "w_gate": mi["w_gate"], "w_up": mi["w_up"], "w_down": mi["w_down"]}
    desc = tp.make_desc(H, I, nq, nkv, d, n_layers=1, seq_len=S_, batch=B, eps=wl.eps)
    x = dev(a["x"], "bf16")
    g1, g2 = dev(a["gamma"], "bf16"), dev(mi["gamma"], "bf16")
    plans = [tp.tp_shard_plan(desc, t, r) for r in range(t)]
    rank_w, caches, attn_parts = [], [], []
    for p in plans:
        kb, kn = p.kv_head_begin, p.kv_heads
        rw = {"attn_norm": g1, "w_qkv": dev(qkv_rank_phys(a, p, d), "bf16"),
              "w_o": dev(phys(a["w_o"][p.q_head_begin * d:(p.q_head_begin + p.q_heads) * d, :]), "bf16"),
              "mlp_norm": g2}
        rw["w_gate"], rw["w_up"], rw["w_down"] = [dev(q, "bf16") for q in mlp_rank_phys(mi, p)]
        kc = dev(a["k_cache"][:, kb:kb + kn], "bf16")
        vc = dev(a["v_cache"][:, kb:kb + kn], "bf16")
        part = empty((B, H), torch.float32)
        tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_ATTN, rw, x, part, kv={"k": kc, "v": vc, "kv_len": S_})
        rank_w.append(rw)
        caches.append((kc, vc))
        attn_parts.append(part)
    h = empty((B, H), torch.bfloat16)
    tp.tp_partial_sum(attn_parts, h, residual=x)
    mlp_parts = []
    for p, rw in zip(plans, rank_w):
        part = empty((B, H), torch.float32)
        tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, rw, h, part)
        mlp_parts.append(part)
    out = empty((B, H), torch.bfloat16)
    tp.tp_partial_sum(mlp_parts, out, residual=h)
    torch.cuda.synchronize()

    say("oracle: unsharded layer")
    ref = L.layer(a["x"], w, a["k_cache"], a["v_cache"], S_, nq, nkv, d, wl.eps)
    for r, p in enumerate(plans):
        kb, kn = p.kv_head_begin, p.kv_heads
        kc, vc = caches[r]
        check(f"rank{r} appended k", host(kc)[:, :, S_ - 1], ref["attn"]["k_cache"][:, kb:kb + kn, S_ - 1],
              TOL["bf16"])
        check(f"rank{r} appended v", host(vc)[:, :, S_ - 1], ref["attn"]["v_cache"][:, kb:kb + kn, S_ - 1],
              TOL["bf16"])
    # every rank's partials against the sharded oracle (its own planner), then their sums before the residual
    odesc = OP.ModelDesc(hidden=H, intermediate=I, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, seq_len=S_, batch=B)
    hh = host(h)
    for r in range(t):
        op = OP.rank_plan(odesc, t, r)
        sr = S.rank_attention(a["x"], a["w_q"], a["w_k"], a["w_v"], a["w_o"], a["k_cache"], a["v_cache"], S_, nq,
                              nkv, d, op, a["gamma"], wl.eps)
        check(f"rank{r} attention partial", host(attn_parts[r]), sr["partial"], TOL["bf16"])
        mr = S.rank_mlp(hh, w["w_gate"], w["w_up"], w["w_down"], op, w["gamma2"], wl.eps)
        check(f"rank{r} MLP partial at the GPU's h", host(mlp_parts[r]), mr["partial"], TOL["bf16"])
    check("sum of 8 attention partials", sum(host(q) for q in attn_parts), ref["attn"]["y"], TOL["bf16"])
    check("h = x + sum of 8 attention partials", hh, ref["h"], TOL["bf16"])
    # the MLP stage against the oracle evaluated at the h the GPU produced
    mref = L.mlp_block(hh, w["w_gate"], w["w_up"], w["w_down"], w["gamma2"], wl.eps)
    mparts = sum(host(q) for q in mlp_parts)
    check("sum of 8 MLP partials at the GPU's h", mparts, mref["y"], TOL["bf16"])
    check("layer output", host(out), ref["out"], TOL["bf16"])


PREFILL_LAYER_CASES = [
    # hidden, intermediate, q heads, kv heads, head_dim, t, sequences, new tokens, kv_len, capacity
    (512, 1024, 8, 2, 64, 2, 2, 4, 9, 16),           # 8 rows: the projections take the GEMV path
    (1024, 2816, 16, 4, 64, 4, 2, 96, 130, 160),     # MFMA GEMMs, a chunk after a cached prefix
    (1024, 2048, 64, 8, 128, 8, 2, 200, 200, 256),   # 70B heads at t=8 (8 q heads on 1 kv head), a prompt
    (512, 1024, 8, 2, 64, 4, 3, 1, 20, 32),          # t > n_kv: kv heads replicated; a decode step
    (512, 1024, 8, 1, 64, 8, 2, 33, 33, 40),         # t = 8 on one kv head (8 copies), a prompt
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", PREFILL_LAYER_CASES, ids=lambda c: "x".join(map(str, c)))
def test_full_layer_prefill_bf16(case):
    """All t rank shards of both stages over a block of new tokens, summed on device, against the oracle."""
    H, I, nq, nkv, d, t, B, S_, kv_len, cap = case
    seed = 60 + t
    a = W.attention_inputs(seed, H, nq, nkv, d, B, cap, "bf16", "random")
    mi = W.mlp_inputs(seed, H, I, 1, "bf16", "random")
    x = W.to_bf16(W.normal(seed, W.Q_PREFILL, (B, S_, H)))
    w = {"gamma1": a["gamma"], "w_q": a["w_q"], "w_k": a["w_k"], "w_v": a["w_v"], "w_o": a["w_o"],
         "gamma2": mi["gamma"], "w_gate": mi["w_gate"], "w_up": mi["w_up"], "w_down": mi["w_down"]}
    desc = tp.make_desc(H, I, nq, nkv, d, n_layers=1, seq_len=cap, batch=B)
    M = B * S_
    xd = dev(x.reshape(M, H), "bf16")
    g1, g2 = dev(a["gamma"], "bf16"), dev(mi["gamma"], "bf16")
    plans = [tp.tp_shard_plan(desc, t, r) for r in range(t)]
    rank_w, caches, attn_parts = [], [], []
    for p in plans:
        kb, kn = p.kv_head_begin, p.kv_heads
        rw = {"attn_norm": g1, "w_qkv": dev(qkv_rank_phys(a, p, d), "bf16"),
              "w_o": dev(phys(a["w_o"][p.q_head_begin * d:(p.q_head_begin + p.q_heads) * d, :]), "bf16"),
              "mlp_norm": g2}
        rw["w_gate"], rw["w_up"], rw["w_down"] = [dev(q, "bf16") for q in mlp_rank_phys(mi, p)]
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

    ref = L.layer_prefill(x, w, a["k_cache"], a["v_cache"], kv_len, nq, nkv, d)
    blk = slice(kv_len - S_, kv_len)
    for r, p in enumerate(plans):
        kb, kn = p.kv_head_begin, p.kv_heads
        kc, vc = caches[r]
        check(f"rank{r} appended k block", host(kc)[:, :, blk], ref["attn"]["k_cache"][:, kb:kb + kn, blk],
              TOL["bf16"])
        check(f"rank{r} appended v block", host(vc)[:, :, blk], ref["attn"]["v_cache"][:, kb:kb + kn, blk],
              TOL["bf16"])
        keep = [j for j in range(cap) if not kv_len - S_ <= j < kv_len]
        assert np.array_equal(host(kc)[:, :, keep], W.to_bf16(a["k_cache"][:, kb:kb + kn][:, :, keep]))
    sr = S.rank_attention_prefill(x, a["w_q"], a["w_k"], a["w_v"], a["w_o"], a["k_cache"], a["v_cache"], kv_len,
                                  nq, nkv, d, tp.plan_dict(plans[-1]), a["gamma"])
    check("last rank attention partial", host(attn_parts[-1]), sr["partial"].reshape(M, H), TOL["bf16"])
    check(f"h = x + sum of {t} attention partials", host(h), ref["h"].reshape(M, H), TOL["bf16"])
    mref = L.mlp_block(host(h), w["w_gate"], w["w_up"], w["w_down"], w["gamma2"])
    check(f"sum of {t} MLP partials at the GPU's h", sum(host(q) for q in mlp_parts), mref["y"], TOL["bf16"])
    check("layer output", host(out), ref["out"].reshape(M, H), TOL["bf16"])


MOE_CASES = [
    # hidden, intermediate (per expert), experts, top_k, t, tokens
    (512, 1024, 4, 2, 2, 5),
    (1024, 2816, 8, 2, 2, 16),
    (1024, 2048, 8, 1, 4, 3),
    # the router's widest expert counts (64 experts, top 8; 32), and more tokens than the fused router
    # launch takes (logits from a projection, gates from their own kernel)
    (256, 256, 64, 8, 2, 7), (256, 512, 32, 2, 1, 33), (256, 512, 16, 4, 2, 80),
]


def moe_inputs(seed, H, I, E, m):
    x = W.to_bf16(W.normal(seed, W.X, (m, H)))
    gamma = W.gamma(seed, W.GAMMA2, H, "random", "bf16")
    w_router = W.to_bf16(W.normal(seed, W.ATTN_IN, (H, E), 0.02))
    experts = []
    for e in range(E):
        mi = W.mlp_inputs(seed * 100 + e, H, I, 1, "bf16")
        experts.append((mi["w_gate"], mi["w_up"], mi["w_down"]))
    return x, gamma, w_router, experts


def moe_rank_phys(experts, p):
    """A rank's stacked expert weights: gate/up [E * cols, H], down [H, E * cols]."""
    b, c = p.inter_begin, p.inter_cols
    wg = np.concatenate([phys(g[:, b:b + c]) for g, _, _ in experts], axis=0)
    wu = np.concatenate([phys(u[:, b:b + c]) for _, u, _ in experts], axis=0)
    wd = np.concatenate([phys(d[b:b + c, :]) for _, _, d in experts], axis=1)
    return wg, wu, wd


@pytest.mark.parametrize("case", MOE_CASES, ids=lambda c: "x".join(map(str, c)))
def test_moe_shard_bf16(case):
    H, I, E, k, t, m = case
    x, gamma, w_router, experts = moe_inputs(70 + E + k, H, I, E, m)
    desc = tp.make_desc(H, I)
    xd, gd, rd = dev(x, "bf16"), dev(gamma, "bf16"), dev(phys(w_router), "bf16")
    parts, gates, logits, plans = [], [], [], []
    for r in range(t):
        p = tp.tp_shard_plan(desc, t, r)
        wg, wu, wd = moe_rank_phys(experts, p)
        w = {"norm": gd, "w_router": rd, "w_gate": dev(wg, "bf16"), "w_up": dev(wu, "bf16"),
             "w_down": dev(wd, "bf16")}
        part = empty((m, H), torch.float32)
        g = empty((m, E), torch.float32)
        lg = empty((m, E), torch.float32)
        tp.tp_moe_shard_forward(w, xd, part, E, k, p.inter_cols, gates=g, logits=lg)
        parts.append(part); gates.append(g); logits.append(lg); plans.append(p)
    out = empty((m, H), torch.float32)
    tp.tp_partial_sum(parts, out)
    torch.cuda.synchronize()
    ref = L.moe_block(x, gamma, w_router, experts, k)
    lg0 = host(logits[0])
    check("router logits", lg0, ref["logits"], TOL["bf16"])
    for r in range(1, t):
        assert np.array_equal(host(gates[r]), host(gates[0])), "ranks disagree on the routing"
    # the routing decision taken in the kernel's precision: top-k of the GPU's logits
    g_ref = L.moe_route(lg0, k)
    g0 = host(gates[0])
    assert np.array_equal(g0 > 0, g_ref > 0), "top-k selection differs"
    assert np.max(np.abs(g0 - g_ref)) < 1e-5
    for r, p in enumerate(plans):
        sr = S.rank_moe(x, gamma, w_router, experts, g0, tp.plan_dict(p))
        check(f"rank{r} MoE partial", host(parts[r]), sr["partial"], TOL["bf16"])
    yref = L.moe_block(x, gamma, w_router, experts, k, gates=g0)["y"]
    check(f"sum of {t} MoE partials", host(out), yref, TOL["bf16"])


@pytest.mark.parametrize("m", [9, 70])
def test_moe_router_ties(m):
    """Experts with identical router rows get identical logits; the lower index wins the tie, on the fused
    router (9 tokens) and on the projection + gates path (70 tokens)."""
    H, I, E, k = 256, 256, 8, 3
    x, gamma, w_router, experts = moe_inputs(91, H, I, E, m)
    w_router = w_router.copy()
    w_router[:, 2] = w_router[:, 1]                  # experts 1 and 2 tie
    w_router[:, 6] = w_router[:, 5]                  # experts 5 and 6 tie
    desc = tp.make_desc(H, I)
    p = tp.tp_shard_plan(desc, 1, 0)
    wg, wu, wd = moe_rank_phys(experts, p)
    w = {"norm": dev(gamma, "bf16"), "w_router": dev(phys(w_router), "bf16"), "w_gate": dev(wg, "bf16"),
         "w_up": dev(wu, "bf16"), "w_down": dev(wd, "bf16")}
    part = empty((m, H), torch.float32)
    g = empty((m, E), torch.float32)
    lg = empty((m, E), torch.float32)
    tp.tp_moe_shard_forward(w, dev(x, "bf16"), part, E, k, p.inter_cols, gates=g, logits=lg)
    torch.cuda.synchronize()
    lg0, g0 = host(lg), host(g)
    assert np.array_equal(lg0[:, 1], lg0[:, 2]) and np.array_equal(lg0[:, 5], lg0[:, 6])
    g_ref = L.moe_route(lg0, k)
    assert np.array_equal(g0 > 0, g_ref > 0), "top-k selection differs"
    assert np.max(np.abs(g0 - g_ref)) < 1e-5
    assert np.all(np.count_nonzero(g0, axis=1) == k)


# ---------------------------------------------------------------- ragged and edge shapes

LINEAR_CASES = [
    # m, k, n, dtype
    (1, 8, 1, "bf16"), (3, 264, 130, "bf16"), (5, 4104, 77, "bf16"), (16, 8200, 300, "bf16"),
    (2, 16384, 64, "bf16"), (9, 1032, 257, "bf16"), (17, 520, 96, "bf16"), (40, 136, 40, "bf16"),
    (1, 4, 3, "f32"), (7, 260, 33, "f32"), (16, 1028, 129, "f32"), (33, 64, 40, "f32"), (4, 6148, 70, "f32"),
    # wide outputs: K split over the 8 waves of one workgroup, ragged n and K, K shorter than one
    # stage, the longest K ranges (8192), and the fallbacks to 64-row tiles split over workgroups
    (16, 4096, 2040, "bf16"), (5, 2056, 6200, "bf16"), (12, 200, 4100, "bf16"), (16, 8200, 6150, "bf16"),
    (16, 8192, 6152, "bf16"), (7, 16384, 2100, "bf16"), (9, 1032, 8200, "bf16"), (5, 17000, 1030, "bf16"),
    # 16-row wide tiles (4096 <= n < 6144 at one block of 16 tokens, or two blocks): the 8B down
    # projection's shape, ragged n with K ending inside a stage, the longest K, K short of one stage per
    # wave, two token blocks
    (16, 3584, 4096, "bf16"), (11, 2040, 5000, "bf16"), (16, 8192, 4104, "bf16"), (6, 136, 6100, "bf16"),
    (20, 1032, 2100, "bf16"),
    # SwiGLU tiles of fewer outputs than rows, sized to fill 256 workgroups (13 outputs, the last tile
    # ragged; 10), and the 70B QKV shard shapes at t=4 and t=8 (K ending inside a stage) that stay on
    # 64-row tiles split over workgroups
    (16, 1032, 3300, "bf16"), (16, 8192, 2560, "bf16"), (16, 4104, 1280, "bf16"), (7, 1032, 1500, "bf16"),
    # 8-wave tiles of 16 to 32 rows with K split over workgroups and merged (where 64-row tiles would
    # stream chunks of 1024 or less): the 70B QKV shard at t=8, ragged n with K ending inside the second
    # split; the t=8 shape at 20 tokens (two token blocks) and at 65 tokens, the first batch on the GEMM
    (16, 8192, 1280, "bf16"), (16, 6000, 2600, "bf16"), (20, 8192, 1280, "bf16"), (65, 8192, 1280, "bf16"),
    # 17 to 64 tokens on the 8-wave GEMV, two token blocks per workgroup: the 70B gate/up, down and W_o
    # shards at t=8 and the 8B down shard at t=4 (16-row tiles); ragged K and n; 16-row tiles at four
    # blocks and, for SwiGLU, at two; a second block of one row (17, 33 tokens) or none (40, 48 tokens)
    (32, 8192, 3584, "bf16"), (40, 3584, 8192, "bf16"), (24, 1024, 8192, "bf16"), (32, 3584, 4096, "bf16"),
    (48, 8136, 2600, "bf16"), (64, 4104, 4096, "bf16"), (56, 2048, 2000, "bf16"), (20, 4096, 2000, "bf16"),
    (17, 2056, 6200, "bf16"), (33, 136, 6100, "bf16"),
    # 17 to 64 tokens stay on the decode GEMV (two to four token blocks) with K of one to three stages
    (17, 8, 67, "bf16"), (20, 24, 130, "bf16"), (18, 64, 300, "bf16"), (64, 96, 260, "bf16"),
    # prefill GEMM with one to three K tiles (the pipeline's prologue alone), ragged and not
    (65, 8, 67, "bf16"), (80, 24, 130, "bf16"), (100, 64, 300, "bf16"), (129, 96, 260, "bf16"),
    (300, 104, 520, "bf16"),
    # outputs of at most 64 (a router's logits) stay on the decode GEMV at any batch: blocks of 16 tokens
    # against one weight tile, K split over workgroups; the Mixtral router's shape at 4096 tokens, the
    # last narrow width and the first on the GEMM
    (4096, 4096, 8, "bf16"), (300, 1032, 64, "bf16"), (300, 1032, 65, "bf16"),
]


@pytest.mark.parametrize("mode", ["col", "col_norm", "swiglu", "swiglu_norm", "row"])
@pytest.mark.parametrize("case", LINEAR_CASES, ids=lambda c: "x".join(map(str, c)))
def test_linear_shapes(case, mode):
    m, k, n, dt = case
    seed = 100 + (31 * m + 7 * k + n) % 1000
    x = W.storage_round(W.normal(seed, 0, (m, k)), dt)
    wp = W.storage_round(W.normal(seed, 1, (n, k), 0.05), dt)     # physical [n, k]
    wu = W.storage_round(W.normal(seed, 2, (n, k), 0.05), dt)
    gam = W.storage_round(W.normal(seed, 3, (k,), 0.1, 1.0), dt)
    norm = mode.endswith("norm")
    u = L.rmsnorm(x, gam, 1e-5) if norm else x.astype(np.float64)
    if mode.startswith("swiglu"):
        ref = L.swiglu(L.linear(u, wp.T), L.linear(u, wu.T))
    else:
        ref = L.linear(u, wp.T)
    tx, tw, twu, tg = dev(x, dt), dev(wp, dt), dev(wu, dt), dev(gam, dt)
    if mode == "row":
        y = empty((m, n), torch.float32)
        tp.tp_row_linear_partial(tx, tw, y)
    else:
        y = empty((m, n), torch.bfloat16 if dt == "bf16" else torch.float32)
        tp.tp_column_linear(tx, tw, y, w_up=twu if mode.startswith("swiglu") else None,
                            gamma=tg if norm else None)
    torch.cuda.synchronize()
    check(f"{mode} m={m} k={k} n={n} {dt}", host(y), ref, TOL[dt])


def _random_linear_cases(n_cases=24, seed=2024, ms=(1, 3, 5, 8, 12, 16, 16, 16, 20, 40)):
    """Seeded shapes across the decode projection kernels (m 1-64) and the GEMM (m above 64): m drawn
    from `ms`, k a multiple of 8 up to 9000, n up to 9000 (work kept small enough for the float64
    reference)."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n_cases:
        m = int(rng.choice(ms))
        k = 8 * int(rng.integers(1, 1126))
        n = int(rng.integers(1, 9001))
        if m * k * n > 1.5e8:
            continue
        mode = ["col", "col_norm", "swiglu", "swiglu_norm", "row"][len(cases) % 5]
        cases.append((m, k, n, mode))
    return cases


@pytest.mark.parametrize("case", _random_linear_cases() + _random_linear_cases(10, 2025, (65, 80, 128, 200)),
                         ids=lambda c: "x".join(map(str, c)))
def test_linear_random_shapes(case):
    m, k, n, mode = case
    seed = 700 + (13 * m + 5 * k + n) % 1000
    x = W.to_bf16(W.normal(seed, 0, (m, k)))
    wp = W.to_bf16(W.normal(seed, 1, (n, k), 0.05))
    wu = W.to_bf16(W.normal(seed, 2, (n, k), 0.05))
    gam = W.to_bf16(W.normal(seed, 3, (k,), 0.1, 1.0))
    norm = mode.endswith("norm")
    u = L.rmsnorm(x, gam, 1e-5) if norm else x.astype(np.float64)
    if mode.startswith("swiglu"):
        ref = L.swiglu(L.linear(u, wp.T), L.linear(u, wu.T))
    else:
        ref = L.linear(u, wp.T)
    tx, tw, twu, tg = dev(x, "bf16"), dev(wp, "bf16"), dev(wu, "bf16"), dev(gam, "bf16")
    if mode == "row":
        y = empty((m, n), torch.float32)
        tp.tp_row_linear_partial(tx, tw, y)
    else:
        y = empty((m, n), torch.bfloat16)
        tp.tp_column_linear(tx, tw, y, w_up=twu if mode.startswith("swiglu") else None, gamma=tg if norm else None)
    torch.cuda.synchronize()
    check(f"{mode} m={m} k={k} n={n}", host(y), ref, TOL["bf16"])


ATTN_CASES = [
    # batch, q_heads, kv_heads, head_dim, capacity, kv_len
    (1, 1, 1, 64, 1, 1), (2, 4, 2, 128, 300, 257), (3, 16, 1, 128, 1000, 1000), (4, 8, 8, 64, 5000, 4097),
    (16, 8, 1, 128, 8192, 8192), (2, 2, 1, 128, 70000, 66000), (5, 4, 4, 128, 256, 255),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "x".join(map(str, c)))
def test_decode_attention_shapes(case):
    B, qh, kvh, d, cap, kv_len = case
    seed = 200 + cap
    q = W.to_bf16(W.normal(seed, 0, (B, qh * d)))
    k = W.to_bf16(W.normal(seed, 1, (B, kvh, cap, d)))
    v = W.to_bf16(W.normal(seed, 2, (B, kvh, cap, d)))
    ref = L.decode_attention(q, k, v, kv_len, qh, kvh, d)
    out = empty((B, qh * d), torch.bfloat16)
    tp.tp_decode_attention(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), out, kv_len, qh)
    torch.cuda.synchronize()
    check(f"attention {case}", host(out), ref, TOL["bf16"])


def test_decode_ignores_cache_past_kv_len():
    """Cache rows at kv_len and beyond hold NaN: no key or value past kv_len may reach the output."""
    B, qh, kvh, d, cap, kv_len = 3, 8, 2, 128, 5000, 4097
    q = W.to_bf16(W.normal(44, 0, (B, qh * d)))
    k = W.to_bf16(W.normal(44, 1, (B, kvh, cap, d)))
    v = W.to_bf16(W.normal(44, 2, (B, kvh, cap, d)))
    ref = L.decode_attention(q, k, v, kv_len, qh, kvh, d)
    k[:, :, kv_len:] = np.nan
    v[:, :, kv_len:] = np.nan
    out = empty((B, qh * d), torch.bfloat16)
    tp.tp_decode_attention(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), out, kv_len, qh)
    torch.cuda.synchronize()
    got = host(out)
    assert np.isfinite(got).all(), "a row past kv_len reached the output"
    check("decode attention with NaN past kv_len", got, ref, TOL["bf16"])


PREFILL_CASES = [
    # batch, q_heads, kv_heads, head_dim, capacity, seq, kv_len
    (1, 1, 1, 64, 1, 1, 1),            # one token, one key
    (1, 1, 1, 128, 5, 1, 5),           # one new token after four cached ones (a decode step)
    (2, 4, 2, 128, 300, 257, 257),     # prompt from scratch, ragged last block
    (3, 2, 2, 64, 130, 130, 130),      # GQ 1: 128 tokens per workgroup, two query blocks
    (1, 16, 1, 64, 600, 100, 555),     # GQ 16: 8 tokens per workgroup, long cached prefix
    (2, 8, 4, 64, 1000, 77, 1000),     # GQ 2, chunk at the end of a full cache
    (2, 8, 1, 128, 3000, 200, 2900),   # 70B t=8 head shard, chunked prefill
    (1, 4, 4, 128, 64, 64, 64),        # GQ 1 with several kv heads, one key block
    (2, 8, 1, 128, 2048, 2048, 2048),  # 70B t=8 head shard at batch 2 x 2048 tokens
    (1, 8, 1, 128, 1000, 128, 640),    # whole key blocks only, cache longer than kv_len
    (1, 16, 1, 64, 128, 5, 128),       # one-token query block ending on a key-block boundary
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "x".join(map(str, c)))
def test_prefill_attention_shapes(case):
    B, qh, kvh, d, cap, S, kv_len = case
    seed = 300 + cap + S
    q = W.to_bf16(W.normal(seed, 0, (B, S, qh * d)))
    k = W.to_bf16(W.normal(seed, 1, (B, kvh, cap, d)))
    v = W.to_bf16(W.normal(seed, 2, (B, kvh, cap, d)))
    ref = L.prefill_attention(q, k, v, kv_len, qh, kvh, d)
    out = torch.full((B, S, qh * d), float("nan"), dtype=torch.bfloat16, device="cuda")
    tp.tp_prefill_attention(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), out, kv_len, qh)
    torch.cuda.synchronize()
    check(f"prefill attention {case}", host(out), ref, TOL["bf16"])


def test_prefill_ignores_cache_past_kv_len():
    """Cache rows at kv_len and beyond hold NaN: no key or value past kv_len may reach the output."""
    B, qh, kvh, d, cap, S, kv_len = 2, 8, 2, 128, 700, 150, 555
    q = W.to_bf16(W.normal(43, 0, (B, S, qh * d)))
    k = W.to_bf16(W.normal(43, 1, (B, kvh, cap, d)))
    v = W.to_bf16(W.normal(43, 2, (B, kvh, cap, d)))
    ref = L.prefill_attention(q, k, v, kv_len, qh, kvh, d)
    kp, vp = k.copy(), v.copy()
    kp[:, :, kv_len:] = np.nan
    vp[:, :, kv_len:] = np.nan
    out = empty((B, S, qh * d), torch.bfloat16)
    tp.tp_prefill_attention(dev(q, "bf16"), dev(kp, "bf16"), dev(vp, "bf16"), out, kv_len, qh)
    torch.cuda.synchronize()
    got = host(out)
    assert np.isfinite(got).all(), "a row past kv_len reached the output"
    check("prefill attention with NaN past kv_len", got, ref, TOL["bf16"])


def test_prefill_last_token_matches_decode():
    """The last token of a prefill block attends to every cached key, as decode does."""
    B, qh, kvh, d, cap, S, kv_len = 4, 8, 1, 128, 1024, 96, 1000
    q = W.to_bf16(W.normal(41, 0, (B, S, qh * d)))
    k = dev(W.to_bf16(W.normal(41, 1, (B, kvh, cap, d))), "bf16")
    v = dev(W.to_bf16(W.normal(41, 2, (B, kvh, cap, d))), "bf16")
    tq = dev(q, "bf16")
    pre = empty((B, S, qh * d), torch.bfloat16)
    tp.tp_prefill_attention(tq, k, v, pre, kv_len, qh)
    dec = empty((B, qh * d), torch.bfloat16)
    tp.tp_decode_attention(tq[:, S - 1].contiguous(), k, v, dec, kv_len, qh)
    torch.cuda.synchronize()
    ref = L.decode_attention(q[:, S - 1], host(k), host(v), kv_len, qh, kvh, d)
    check("prefill last token", host(pre)[:, S - 1], ref, TOL["bf16"])
    check("decode of the same token", host(dec), ref, TOL["bf16"])


def _random_attention_cases(n_cases=16, seed=2025, prefill=False):
    """Seeded attention shapes: group sizes 1-16, 1-4 kv heads, both head sizes, caches longer than
    kv_len; decode up to 20,000 keys at batch 1-24, prefill blocks of 1-700 tokens after a cached prefix
    of up to 800 (work kept small enough for the float64 reference)."""
    rng = np.random.default_rng(seed + int(prefill))
    cases = []
    while len(cases) < n_cases:
        gq = int(rng.choice([1, 2, 4, 8, 16]))
        kvh = int(rng.choice([1, 1, 2, 4]))
        d = int(rng.choice([64, 128]))
        if prefill:
            B = int(rng.integers(1, 4))
            S = int(rng.integers(1, 701))
            kv_len = S + int(rng.integers(0, 801))
            if B * gq * kvh * S * kv_len * d > 2e9:
                continue
        else:
            B = int(rng.integers(1, 25))
            S = 1
            kv_len = int(rng.integers(1, 20001))
        cap = kv_len + int(rng.integers(0, 301))
        if not prefill and (B * gq * kvh * kv_len * d > 1e9 or B * kvh * cap * d > 2e7):
            continue
        cases.append((B, gq * kvh, kvh, d, cap, S, kv_len))
    return cases


@pytest.mark.parametrize("case", _random_attention_cases(), ids=lambda c: "x".join(map(str, c)))
def test_decode_attention_random_shapes(case):
    B, qh, kvh, d, cap, _, kv_len = case
    seed = 900 + (7 * B + 3 * cap + kv_len) % 1000
    q = W.to_bf16(W.normal(seed, 0, (B, qh * d)))
    k = W.to_bf16(W.normal(seed, 1, (B, kvh, cap, d)))
    v = W.to_bf16(W.normal(seed, 2, (B, kvh, cap, d)))
    ref = L.decode_attention(q, k, v, kv_len, qh, kvh, d)
    out = torch.full((B, qh * d), float("nan"), dtype=torch.bfloat16, device="cuda")
    tp.tp_decode_attention(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), out, kv_len, qh)
    torch.cuda.synchronize()
    check(f"decode attention {case}", host(out), ref, TOL["bf16"])


@pytest.mark.parametrize("case", _random_attention_cases(prefill=True), ids=lambda c: "x".join(map(str, c)))
def test_prefill_attention_random_shapes(case):
    B, qh, kvh, d, cap, S, kv_len = case
    seed = 950 + (7 * B + 3 * cap + S) % 1000
    q = W.to_bf16(W.normal(seed, 0, (B, S, qh * d)))
    k = W.to_bf16(W.normal(seed, 1, (B, kvh, cap, d)))
    v = W.to_bf16(W.normal(seed, 2, (B, kvh, cap, d)))
    ref = L.prefill_attention(q, k, v, kv_len, qh, kvh, d)
    out = torch.full((B, S, qh * d), float("nan"), dtype=torch.bfloat16, device="cuda")
    tp.tp_prefill_attention(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), out, kv_len, qh)
    torch.cuda.synchronize()
    check(f"prefill attention {case}", host(out), ref, TOL["bf16"])


@pytest.mark.parametrize("t", [1, 3, 8])
@pytest.mark.parametrize("shape", [(5, 7), (16, 8192), (3, 1)])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
@pytest.mark.parametrize("residual", [False, True])
def test_partial_sum_shapes(t, shape, out_dt, residual):
    parts = [W.normal(300 + r, 0, shape) for r in range(t)]
    res = W.storage_round(W.normal(399, 0, shape), out_dt) if residual else None
    ref = sum(p.astype(np.float64) for p in parts) + (res if residual else 0.0)
    out = empty(shape, torch.bfloat16 if out_dt == "bf16" else torch.float32)
    tp.tp_partial_sum([dev(p, "f32") for p in parts], out, residual=dev(res, out_dt) if residual else None)
    torch.cuda.synchronize()
    check(f"partial sum t={t} {shape} {out_dt}", host(out), ref, 1e-6 if out_dt == "f32" else 2 ** -8)


@pytest.mark.parametrize("t", [1, 3, 8])
@pytest.mark.parametrize("shape", [(5, 7), (16, 8192), (3, 1)])
@pytest.mark.parametrize("out_dt", ["f32", "bf16"])
@pytest.mark.parametrize("residual", [False, True])
def test_partial_sum_bf16_shapes(t, shape, out_dt, residual):
    parts = [W.to_bf16(W.normal(300 + r, 0, shape)) for r in range(t)]
    res = W.storage_round(W.normal(399, 0, shape), out_dt) if residual else None
    ref = sum(p.astype(np.float64) for p in parts) + (res if residual else 0.0)
    out = empty(shape, torch.bfloat16 if out_dt == "bf16" else torch.float32)
    tp.tp_partial_sum_bf16([dev(p, "bf16") for p in parts], out, residual=dev(res, out_dt) if residual else None)
    torch.cuda.synchronize()
    check(f"bf16 partial sum t={t} {shape} {out_dt}", host(out), ref, 1e-6 if out_dt == "f32" else 2 ** -8)


@pytest.mark.parametrize("case", [c for c in LINEAR_CASES if c[3] == "bf16"], ids=lambda c: "x".join(map(str, c)))
def test_row_partial_bf16_shapes(case):
    m, k, n, _ = case
    seed = 500 + m + k
    x = W.to_bf16(W.normal(seed, 0, (m, k)))
    wl_ = W.to_bf16(W.normal(seed, 1, (k, n), 0.02))
    ref = L.linear(x, wl_)
    part = empty((m, n), torch.bfloat16)
    tp.tp_row_linear_partial_bf16(dev(x, "bf16"), dev(phys(wl_), "bf16"), part)
    torch.cuda.synchronize()
    check(f"bf16 row partial m={m} k={k} n={n}", host(part), ref, TOL["bf16"])


@pytest.mark.parametrize("count", [(1, 1), (3, 333), (16, 3584)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_swiglu_standalone(count, dt):
    g = W.storage_round(W.normal(400, 0, count, 3.0), dt)
    u = W.storage_round(W.normal(400, 1, count), dt)
    out = empty(count, torch.bfloat16 if dt == "bf16" else torch.float32)
    tp.tp_swiglu(dev(g, dt), dev(u, dt), out)
    torch.cuda.synchronize()
    check(f"swiglu {count} {dt}", host(out), L.swiglu(g, u), TOL[dt])


def test_repeatable_and_workspace_reuse():
    """Same inputs, same workspace, twice: bitwise identical (split-K counters reset)."""
    m, k, n = 16, 8192, 1280
    x = dev(W.to_bf16(W.normal(500, 0, (m, k))), "bf16")
    w = dev(W.to_bf16(W.normal(500, 1, (n, k), 0.02)), "bf16")
    g = dev(W.to_bf16(W.normal(500, 2, (k,), 0.1, 1.0)), "bf16")
    ws = tp.workspace(tp.tp_linear_workspace_bytes(m, k, n, tp.TP_BF16, tp.TP_LINEAR_NORM))
    ys = []
    for _ in range(3):
        y = empty((m, n), torch.bfloat16)
        tp.tp_column_linear(x, w, y, gamma=g, ws=ws)
        ys.append(y)
    q = dev(W.to_bf16(W.normal(501, 0, (16, 8 * 128))), "bf16")
    kc = dev(W.to_bf16(W.normal(501, 1, (16, 1, 8192, 128))), "bf16")
    vc = dev(W.to_bf16(W.normal(501, 2, (16, 1, 8192, 128))), "bf16")
    aws = tp.workspace(tp.tp_attention_workspace_bytes(16, 8, 1, 128, 8192))
    outs = []
    for _ in range(3):
        o = empty((16, 8 * 128), torch.bfloat16)
        tp.tp_decode_attention(q, kc, vc, o, 8192, 8, ws=aws)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    for w_ in (ws, aws):
        wp, _ = tp._ws(w_)
        off = wp - w_.data_ptr()
        assert int(w_[off:off + 32768].sum()) == 0, "counter header not left zero"


def test_workspace_shared_across_shapes():
    """One workspace, sized for the largest call, serves calls of different shapes in turn."""
    cases = [(16, 8192, 1280, "col"), (16, 1024, 8192, "row"), (4, 4096, 7168, "col"), (16, 3584, 4096, "row"),
             (1, 8192, 300, "col")]
    need = max(tp.tp_linear_workspace_bytes(m, k, n, tp.TP_BF16, tp.TP_LINEAR_NORM) for m, k, n, _ in cases)
    ws = tp.workspace(need)
    for rep in range(2):
        for i, (m, k, n, kind) in enumerate(cases):
            x = W.to_bf16(W.normal(600 + i, 0, (m, k)))
            w = W.to_bf16(W.normal(600 + i, 1, (n, k), 0.02))
            if kind == "row":
                y = empty((m, n), torch.float32)
                tp.tp_row_linear_partial(dev(x, "bf16"), dev(w, "bf16"), y, ws=ws)
            else:
                y = empty((m, n), torch.bfloat16)
                tp.tp_column_linear(dev(x, "bf16"), dev(w, "bf16"), y, ws=ws)
            torch.cuda.synchronize()
            check(f"shared workspace {kind} m={m} k={k} n={n} pass {rep}", host(y), L.linear(x, w.T), TOL["bf16"])
    wp, _ = tp._ws(ws)
    off = wp - ws.data_ptr()
    assert int(ws[off:off + 32768].sum()) == 0, "counter header not left zero"
