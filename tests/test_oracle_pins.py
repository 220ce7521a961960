"""The oracle against its pins (CPU only)."""
import oracle_pins as P
from oracle import layer as L
from oracle import plan
from oracle import sharded as S


def test_kv_worked_example():
    P.pin_kv_worked_example(plan.kv_elements_per_sequence, plan.kv_bytes_per_gpu)


def test_weight_footprint():
    P.pin_weight_footprint(plan.weight_bytes_per_gpu)


def test_head_blocks():
    P.pin_head_blocks(plan.rank_plan, plan.ModelDesc)


def test_workload_shapes():
    P.pin_workload_shapes(plan.rank_plan, plan.ModelDesc)


def test_plan_errors():
    P.pin_plan_errors(plan.rank_plan, plan.ModelDesc, plan.PlanError)


def test_silu_layer():
    P.pin_silu(L.silu)


def test_silu_sharded():
    P.pin_silu(S._silu)


def test_rmsnorm_layer():
    P.pin_rmsnorm(L.rmsnorm)


def test_rmsnorm_sharded():
    P.pin_rmsnorm(lambda x, g, eps: S._norm(x, g, eps))


def test_mlp_vs_naive():
    P.pin_mlp_vs_naive(L.mlp_block)


def test_attention_vs_naive():
    P.pin_attention_vs_naive(L.decode_attention)


def test_attention_special_cases():
    P.pin_attention_special_cases(L.decode_attention)


def test_column_concat_bitwise():
    P.pin_column_concat_naive(S.column_shard, plan.rank_plan, plan.ModelDesc)


def test_row_partials_sum():
    P.pin_row_partials_sum(S.row_shard, S.sum_partials, plan.rank_plan, plan.ModelDesc)


def test_sharded_mlp_matches_unsharded():
    P.pin_sharded_mlp(S.sharded_mlp, L.mlp_block)


def test_sharded_layer_matches_unsharded():
    P.pin_sharded_layer(S.sharded_layer, L.layer)


def test_layer_literal_flow():
    P.pin_layer_literal_flow(L.layer, L.attention_block, L.mlp_block)


def test_layer_vs_naive():
    P.pin_layer_vs_naive(L.layer)


def test_prefill_attention():
    P.pin_prefill_attention(L.prefill_attention, L.decode_attention)


def test_rank_prefill_attention():
    P.pin_rank_prefill(S.rank_prefill_attention, L.prefill_attention, plan.rank_plan, plan.ModelDesc)


def test_layer_prefill_one_token():
    P.pin_layer_prefill_one_token(L.layer_prefill, L.layer)


def test_layer_prefill_chunks():
    P.pin_layer_prefill_chunks(L.layer_prefill)


def test_layer_prefill_vs_naive():
    P.pin_layer_prefill_vs_naive(L.layer_prefill)


def test_sharded_layer_prefill():
    P.pin_sharded_layer_prefill(S.sharded_layer_prefill, L.layer_prefill)


def test_moe_route():
    P.pin_moe_route(L.moe_route)


def test_moe_identical_and_single():
    P.pin_moe_identical_and_single(L.moe_block, L.mlp_block)


def test_moe_vs_naive():
    P.pin_moe_vs_naive(L.moe_block)


def test_rank_moe():
    P.pin_rank_moe(S.rank_moe, L.moe_block, plan.rank_plan, plan.ModelDesc)


def test_kv_replication():
    P.pin_kv_replication(plan.rank_plan, plan.ModelDesc)



def test_attn_proj_block():
    P.pin_attn_proj_block(L.attn_proj_block)


def test_layer_weight_elements():
    P.pin_layer_weight_elements(plan.layer_weight_elements, plan.rank_plan, plan.ModelDesc)
