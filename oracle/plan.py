"""Integer shard planner and memory footprints (oracle side).

Sources:
- "Tensor parallel scaling curves", section "What tensor parallelism actually
  splits": Q, K, V are split by columns so that each GPU owns a subset of the
  attention heads, given as the contiguous block heads[rank*h_per_gpu :
  (rank+1)*h_per_gpu]; the output projection is split by rows; the MLP gate and
  up projections by columns and the down projection by rows.
- "Tensor Parallelism Fundamentals", section "Memory Overhead and Communication
  Bottlenecks": weights and KV cache per GPU are the totals divided by t; the KV
  bytes per GPU are 2 x layers x kv_heads x head_dim x seq_length x
  bytes_per_element x batch / t.
- "Tensor Parallelism" (Lifeboat docs) and "Tensor Parallelism Fundamentals",
  section "Sizing Heuristics and Limits": t lies in 1..8.

Readings where the pages are silent: intermediate columns are assigned in the
same contiguous rank order as heads; gate and up share one column block so the
gating stays local to the rank; t must divide the q heads, the kv heads and the
intermediate size (no replication, no uneven split).
"""
from __future__ import annotations

import dataclasses


class PlanError(ValueError):
    """Invalid plan request. ``kind`` is 'RANK', 'SHAPE' or 'INDIVISIBLE'."""

    def __init__(self, kind: str, msg: str):
        super().__init__(msg)
        self.kind = kind


@dataclasses.dataclass(frozen=True)
class ModelDesc:
    hidden: int
    intermediate: int = 0        # 0: no MLP
    n_q_heads: int = 0           # 0: no attention
    n_kv_heads: int = 0
    head_dim: int = 0
    n_layers: int = 1
    seq_len: int = 0             # KV length per sequence (footprint only)
    batch: int = 1
    bytes_per_elem: int = 2


def kv_elements_per_sequence(n_layers: int, n_kv_heads: int, head_dim: int, seq_len: int) -> int:
    """Keys and values of one sequence across all layers: 2 * L * kv_heads * d * S."""
    return 2 * n_layers * n_kv_heads * head_dim * seq_len


def kv_bytes_per_gpu(n_layers: int, n_kv_heads: int, head_dim: int, seq_len: int,
                     bytes_per_elem: int, batch: int, t: int) -> int:
    """KV bytes one GPU holds: the whole batch's KV bytes divided by t (exact when t | kv_heads)."""
    total = kv_elements_per_sequence(n_layers, n_kv_heads, head_dim, seq_len) * bytes_per_elem * batch
    if total % t:
        raise PlanError("INDIVISIBLE", f"KV bytes {total} not divisible by t={t}")
    return total // t


def weight_bytes_per_gpu(total_weight_bytes: int, t: int) -> int:
    """Static weight bytes per GPU: the total divided by t."""
    if total_weight_bytes % t:
        raise PlanError("INDIVISIBLE", f"{total_weight_bytes} bytes not divisible by t={t}")
    return total_weight_bytes // t


def layer_weight_elements(desc: ModelDesc) -> int:
    """Unsharded projection weights of one layer (norm scales excluded)."""
    H, d = desc.hidden, desc.head_dim
    attn = H * (desc.n_q_heads + 2 * desc.n_kv_heads) * d + desc.n_q_heads * d * H
    mlp = 3 * H * desc.intermediate
    return attn + mlp


def rank_plan(desc: ModelDesc, t: int, rank: int) -> dict:
    """What rank ``rank`` of ``t`` owns: head blocks, intermediate block, shapes, footprints."""
    if not 1 <= t <= 8:
        raise PlanError("RANK", f"t={t} outside 1..8")
    if not 0 <= rank < t:
        raise PlanError("RANK", f"rank={rank} outside 0..{t - 1}")
    if desc.hidden <= 0 or desc.intermediate < 0 or desc.n_q_heads < 0:
        raise PlanError("SHAPE", "hidden must be > 0; intermediate and heads >= 0")
    has_attn = desc.n_q_heads > 0
    if has_attn:
        if desc.n_kv_heads <= 0 or desc.head_dim <= 0:
            raise PlanError("SHAPE", "attention needs n_kv_heads > 0 and head_dim > 0")
        if desc.n_q_heads % desc.n_kv_heads:
            raise PlanError("INDIVISIBLE", "n_q_heads must be a multiple of n_kv_heads")
        if desc.n_q_heads % t:
            raise PlanError("INDIVISIBLE", f"t={t} must divide q heads {desc.n_q_heads}")
        if desc.n_kv_heads % t and t % desc.n_kv_heads:
            raise PlanError("INDIVISIBLE", f"t={t} must divide, or be a multiple of, kv heads {desc.n_kv_heads}")
    if desc.intermediate % t:
        raise PlanError("INDIVISIBLE", f"t={t} must divide intermediate {desc.intermediate}")

    q_r = desc.n_q_heads // t if has_attn else 0
    # t > n_kv: every rank keeps the one kv head its q heads read (t / n_kv copies of each).
    replicate = has_attn and desc.n_kv_heads % t != 0
    kv_r = (1 if replicate else desc.n_kv_heads // t) if has_attn else 0
    kv_begin = (rank // (t // desc.n_kv_heads) if replicate else rank * kv_r) if has_attn else 0
    i_r = desc.intermediate // t
    d = desc.head_dim if has_attn else 0
    H = desc.hidden
    weight_elems = H * (q_r + 2 * kv_r) * d + q_r * d * H + 3 * H * i_r
    kv_seq = kv_elements_per_sequence(desc.n_layers, desc.n_kv_heads, d, desc.seq_len) if has_attn else 0
    if not has_attn:
        kv_rank = 0
    elif replicate:
        # one kv head's cache: the total divided by n_kv, not by t
        kv_rank = kv_elements_per_sequence(desc.n_layers, 1, d, desc.seq_len) * desc.bytes_per_elem * desc.batch
    else:
        kv_rank = kv_bytes_per_gpu(desc.n_layers, desc.n_kv_heads, d, desc.seq_len, desc.bytes_per_elem,
                                   desc.batch, t)
    return {
        "t": t,
        "rank": rank,
        "q_head_begin": rank * q_r,
        "q_heads": q_r,
        "kv_head_begin": kv_begin,
        "kv_heads": kv_r,
        "inter_begin": rank * i_r,
        "inter_cols": i_r,
        "qkv_cols": (q_r + 2 * kv_r) * d,
        "o_rows": q_r * d,
        "weight_elems": weight_elems,
        "kv_elems_per_seq_all_layers": kv_seq,
        "kv_bytes_rank": kv_rank,
    }
