"""The allocation-free layer entry point (tp_layer_shard_forward_static) against
the workspace entry point (tp_layer_shard_forward) through the C ABI.

Both stages of one rank shard, twice in a row on the same GPU: first 16
sequences (matrix-core decode projections), then 1 (the v_dot2 projections,
whose split-K completion counters live in the static scratch's header). The
two entry points run the same kernels, so their outputs must agree bitwise;
both are also checked against the float64 oracle (2e-2 of max |ref|).
"""
import numpy as np
import pytest
import torch

import megatron_tensor_transformer_amd as tp
import workloads as W
from gpu_helpers import TOL, check, dev, host, phys, say
from oracle import plan as OP
from oracle import sharded as S

pytestmark = pytest.mark.gpu

H, I, NQ, NKV, D, T, CAP, KV_LEN, RANK = 2048, 5632, 16, 4, 128, 2, 700, 650, 1


def _rank_weights(a, mi, p):
    qb, qn, kb, kn = p.q_head_begin, p.q_heads, p.kv_head_begin, p.kv_heads
    wqkv = np.concatenate([phys(a["w_q"][:, qb * D:(qb + qn) * D]), phys(a["w_k"][:, kb * D:(kb + kn) * D]),
                           phys(a["w_v"][:, kb * D:(kb + kn) * D])], axis=0)
    b, c = p.inter_begin, p.inter_cols
    return {"attn_norm": dev(a["gamma"], "bf16"), "w_qkv": dev(wqkv, "bf16"),
            "w_o": dev(phys(a["w_o"][qb * D:(qb + qn) * D, :]), "bf16"), "mlp_norm": dev(mi["gamma"], "bf16"),
            "w_gate": dev(phys(mi["w_gate"][:, b:b + c]), "bf16"), "w_up": dev(phys(mi["w_up"][:, b:b + c]), "bf16"),
            "w_down": dev(phys(mi["w_down"][b:b + c, :]), "bf16")}


@pytest.mark.parametrize("batches", [(16, 1)])
def test_static_scratch_matches_workspace_entry(batches):
    assert torch.cuda.is_available()
    for call, B in enumerate(batches):
        say(f"call {call}: batch {B}")
        a = W.attention_inputs(90 + B, H, NQ, NKV, D, B, CAP, "bf16", "random")
        mi = W.mlp_inputs(90 + B, H, I, B, "bf16", "random")
        desc = tp.make_desc(H, I, NQ, NKV, D, n_layers=1, seq_len=CAP, batch=B)
        p = tp.tp_shard_plan(desc, T, RANK)
        rw = _rank_weights(a, mi, p)
        kb, kn = p.kv_head_begin, p.kv_heads
        x = dev(a["x"], "bf16")
        outs = {}
        for name in ("workspace", "static"):
            kc = dev(a["k_cache"][:, kb:kb + kn], "bf16")
            vc = dev(a["v_cache"][:, kb:kb + kn], "bf16")
            pa = torch.empty(B, H, dtype=torch.float32, device="cuda")
            pm = torch.empty(B, H, dtype=torch.float32, device="cuda")
            h = (x.float() + 0.5).to(torch.bfloat16)    # an MLP input of the right shape
            kv = {"k": kc, "v": vc, "kv_len": KV_LEN}
            if name == "workspace":
                tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_ATTN, rw, x, pa, kv=kv)
                tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, rw, h, pm)
            else:
                tp.tp_layer_shard_forward_static(desc, p, tp.TP_STAGE_ATTN, rw, x, pa, kv=kv)
                tp.tp_layer_shard_forward_static(desc, p, tp.TP_STAGE_MLP, rw, h, pm)
            torch.cuda.synchronize()
            outs[name] = {"attn": host(pa), "mlp": host(pm), "k": host(kc), "v": host(vc), "h": host(h)}
        for key in ("attn", "mlp", "k", "v"):
            assert np.array_equal(outs["static"][key], outs["workspace"][key]), (call, key)
        op = OP.rank_plan(OP.ModelDesc(hidden=H, intermediate=I, n_q_heads=NQ, n_kv_heads=NKV, head_dim=D,
                                       seq_len=CAP, batch=B), T, RANK)
        sr = S.rank_attention(a["x"], a["w_q"], a["w_k"], a["w_v"], a["w_o"], a["k_cache"], a["v_cache"], KV_LEN,
                              NQ, NKV, D, op, a["gamma"])
        check(f"call {call} static attention partial", outs["static"]["attn"], sr["partial"], TOL["bf16"])
        mr = S.rank_mlp(outs["static"]["h"], mi["w_gate"], mi["w_up"], mi["w_down"], op, mi["gamma"])
        check(f"call {call} static MLP partial", outs["static"]["mlp"], mr["partial"], TOL["bf16"])
