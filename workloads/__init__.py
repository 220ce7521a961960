"""Seeded synthetic inputs and the workload shapes they are drawn for.

This module is the only code that both the CPU oracle and the HIP path's tests
use. It holds no arithmetic of the layer itself: it draws normal variates from
a seeded generator, rounds them to the storage precision the GPU receives, and
records the shapes of the measured workloads.

Seeding: every tensor is drawn from ``numpy.random.default_rng([workload_id,
tensor_id])`` with ``standard_normal(dtype=float32)`` and then scaled by its
standard deviation in float32. Every weight is drawn *unsharded*, in the
logical ``[in, out]`` orientation used by ``x @ W`` ("Tensor parallel scaling
curves", section "What tensor parallelism actually splits"); each side slices
it per rank with its own planner, so a slicing mistake on either side shows up
as a parity failure.

"N(0, 0.02)" is read as a standard deviation of 0.02.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence

import numpy as np

# Tensor ids (second seed word).
X, GAMMA1, W_Q, W_K, W_V, W_O, GAMMA2, W_GATE, W_UP, W_DOWN, K_CACHE, V_CACHE, ATTN_IN, Q_PREFILL = range(14)

WEIGHT_STD = 0.02


def normal(workload_id: int, tensor_id: int, shape: Sequence[int], std: float = 1.0,
           mean: float = 0.0) -> np.ndarray:
    """float32 array of N(mean, std^2) draws, seeded by (workload_id, tensor_id)."""
    rng = np.random.default_rng([int(workload_id), int(tensor_id)])
    a = rng.standard_normal(tuple(int(s) for s in shape), dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns of a float32 array, round-to-nearest-even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """float32 array holding the exact values of uint16 bfloat16 bit patterns."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array whose values are a rounded to bfloat16 (round-to-nearest-even)."""
    return from_bf16_bits(bf16_bits(a))


def storage_round(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float32 array to the storage precision 'f32' or 'bf16' (kept as float32)."""
    if dtype == "bf16":
        return to_bf16(a)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one workload. Sizes are unsharded unless the name says per rank."""
    workload_id: int
    name: str
    dtype: str                 # 'f32' or 'bf16' storage
    hidden: int
    intermediate: int          # 0: no MLP
    t: int
    tokens: Sequence[int]      # M values (decode batch or prefill rows)
    n_q_heads: int = 0         # 0: no attention
    n_kv_heads: int = 0
    head_dim: int = 0
    kv_len: int = 0            # cached keys attended over (decode attention)
    norm: bool = False         # RMSNorm in front of the column projections
    eps: float = 1e-5
    attn_proj_only: bool = False   # QKV column + W_o row partial, no attention between

    @property
    def q_cols(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_cols(self) -> int:
        return self.n_kv_heads * self.head_dim


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "tiny MLP block, fp32, hidden 256, intermediate 1024, t=2, 4 tokens",
                "f32", hidden=256, intermediate=1024, t=2, tokens=(4,)),
    2: Workload(2, "Llama-3-8B-shaped MLP decode shard, bf16, hidden 4096, intermediate 14336, t=4",
                "bf16", hidden=4096, intermediate=14336, t=4, tokens=(1, 4, 16), norm=True),
    3: Workload(3, "70B-shaped attention projection decode shard, bf16, hidden 8192, 64 q / 8 kv heads, t=4",
                "bf16", hidden=8192, intermediate=0, t=4, tokens=(16,), n_q_heads=64, n_kv_heads=8,
                head_dim=128, attn_proj_only=True),
    4: Workload(4, "70B-shaped MLP prefill shard, bf16, hidden 8192, intermediate 28672, t=4, 4096 tokens",
                "bf16", hidden=8192, intermediate=28672, t=4, tokens=(4096,)),
    5: Workload(5, "70B-shaped full layer decode shard, bf16, t=8, batch 16, KV 8192",
                "bf16", hidden=8192, intermediate=28672, t=8, tokens=(16,), n_q_heads=64, n_kv_heads=8,
                head_dim=128, kv_len=8192, norm=True),
    6: Workload(6, "70B-shaped causal prefill attention shard, bf16, t=8, batch 2 x 2048 tokens",
                "bf16", hidden=8192, intermediate=0, t=8, tokens=(4096,), n_q_heads=64, n_kv_heads=8,
                head_dim=128, kv_len=2048),
    8: Workload(8, "Mixtral-8x7B-shaped MoE FFN decode shard, bf16, hidden 4096, 8 experts x intermediate "
                   "14336, top-2, t=2, 16 tokens", "bf16", hidden=4096, intermediate=14336, t=2, tokens=(16,),
                norm=True),
    9: Workload(9, "Mixtral-8x7B-shaped MoE FFN prefill shard, bf16, hidden 4096, 8 experts x intermediate "
                   "14336, top-2, t=2, 4096 tokens", "bf16", hidden=4096, intermediate=14336, t=2, tokens=(4096,),
                norm=True),
    7: Workload(7, "70B-shaped full layer prefill shard, bf16, t=8, batch 2 x 2048 tokens",
                "bf16", hidden=8192, intermediate=28672, t=8, tokens=(4096,), n_q_heads=64, n_kv_heads=8,
                head_dim=128, kv_len=2048, norm=True),
}


def gamma(workload_id: int, tensor_id: int, n: int, mode: str, dtype: str) -> np.ndarray:
    """RMSNorm scale: all ones ('ones') or 1 + 0.1 N(0,1) ('random'), storage-rounded."""
    if mode == "ones":
        return np.ones(n, np.float32)
    if mode == "random":
        return storage_round(normal(workload_id, tensor_id, (n,), std=0.1, mean=1.0), dtype)
    raise ValueError(mode)


def mlp_inputs(workload_id: int, hidden: int, intermediate: int, m: int, dtype: str,
               gamma_mode: Optional[str] = None) -> Dict[str, np.ndarray]:
    """x [m, H], W_gate/W_up [H, I], W_down [I, H] (logical), optional gamma [H]."""
    out = {
        "x": storage_round(normal(workload_id, X, (m, hidden)), dtype),
        "w_gate": storage_round(normal(workload_id, W_GATE, (hidden, intermediate), WEIGHT_STD), dtype),
        "w_up": storage_round(normal(workload_id, W_UP, (hidden, intermediate), WEIGHT_STD), dtype),
        "w_down": storage_round(normal(workload_id, W_DOWN, (intermediate, hidden), WEIGHT_STD), dtype),
    }
    if gamma_mode is not None:
        out["gamma"] = gamma(workload_id, GAMMA2, hidden, gamma_mode, dtype)
    return out


def attention_inputs(workload_id: int, hidden: int, n_q: int, n_kv: int, d: int, batch: int,
                     capacity: int, dtype: str, gamma_mode: Optional[str] = None,
                     with_cache: bool = True) -> Dict[str, np.ndarray]:
    """x [B, H]; W_q [H, n_q d], W_k/W_v [H, n_kv d], W_o [n_q d, H]; K/V caches [B, n_kv, capacity, d]."""
    out = {
        "x": storage_round(normal(workload_id, X, (batch, hidden)), dtype),
        "w_q": storage_round(normal(workload_id, W_Q, (hidden, n_q * d), WEIGHT_STD), dtype),
        "w_k": storage_round(normal(workload_id, W_K, (hidden, n_kv * d), WEIGHT_STD), dtype),
        "w_v": storage_round(normal(workload_id, W_V, (hidden, n_kv * d), WEIGHT_STD), dtype),
        "w_o": storage_round(normal(workload_id, W_O, (n_q * d, hidden), WEIGHT_STD), dtype),
    }
    if with_cache:
        out["k_cache"] = storage_round(normal(workload_id, K_CACHE, (batch, n_kv, capacity, d)), dtype)
        out["v_cache"] = storage_round(normal(workload_id, V_CACHE, (batch, n_kv, capacity, d)), dtype)
    if gamma_mode is not None:
        out["gamma"] = gamma(workload_id, GAMMA1, hidden, gamma_mode, dtype)
    return out


def attn_proj_input(workload_id: int, m: int, cols: int, dtype: str) -> np.ndarray:
    """Synthetic attention output fed to W_o when no attention runs in between."""
    return storage_round(normal(workload_id, ATTN_IN, (m, cols)), dtype)


def prefill_attention_inputs(workload_id: int, batch: int, seq: int, n_q: int, n_kv: int, d: int,
                             capacity: int, dtype: str) -> Dict[str, np.ndarray]:
    """q [B, seq, n_q d] for a block of new tokens; K/V caches [B, n_kv, capacity, d]; all N(0, 1)."""
    return {
        "q": storage_round(normal(workload_id, Q_PREFILL, (batch, seq, n_q * d)), dtype),
        "k_cache": storage_round(normal(workload_id, K_CACHE, (batch, n_kv, capacity, d)), dtype),
        "v_cache": storage_round(normal(workload_id, V_CACHE, (batch, n_kv, capacity, d)), dtype),
    }


MOE_EXPERTS, MOE_TOP_K = 8, 2       # the Mixtral-8x7B routing: 8 experts, the top 2 per token


def moe_inputs(workload_id: int, hidden: int, intermediate: int, n_experts: int, m: int,
               dtype: str, progress=None) -> Dict[str, object]:
    """x [m, H], gamma [H] (1 + 0.1 N(0,1)), router [H, E] N(0, 0.02), and per expert the logical
    (w_gate [H, I], w_up [H, I], w_down [I, H]) drawn as an MLP of its own seed. ``progress(e)`` is
    called after each expert is drawn."""
    experts = []
    for e in range(n_experts):
        mi = mlp_inputs(workload_id * 100 + e, hidden, intermediate, 1, dtype)
        experts.append((mi["w_gate"], mi["w_up"], mi["w_down"]))
        if progress is not None:
            progress(e)
    return {
        "x": storage_round(normal(workload_id, X, (m, hidden)), dtype),
        "gamma": gamma(workload_id, GAMMA2, hidden, "random", dtype),
        "w_router": storage_round(normal(workload_id, ATTN_IN, (hidden, n_experts), WEIGHT_STD), dtype),
        "experts": experts,
    }

