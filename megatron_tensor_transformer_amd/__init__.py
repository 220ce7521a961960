"""Python binding of libtpshard.so: one GPU's shard of a Megatron-style
tensor-parallel transformer layer on MI355X (gfx950).

The functions here carry the C entry points' names and only marshal
arguments: torch tensors become device pointers and sizes, the current torch
stream becomes the hipStream_t, and a non-OK status becomes ``TPError``. Every
step of the computation runs in the library's HIP kernels; there is no other
code path. Importing this package fails if the library has not been built.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already mapped (both carry the soname libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtpshard.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python megatron_tensor_transformer_amd/build.py` "
                      "(or __graft_entry__.build()) first")

lib = ctypes.CDLL(LIB_PATH)

TP_F32, TP_BF16 = 0, 1
TP_STAGE_ATTN, TP_STAGE_MLP = 0, 1
TP_LINEAR_SWIGLU, TP_LINEAR_NORM = 1, 2

STATUS = ["TP_OK", "TP_ERR_NULL", "TP_ERR_SHAPE", "TP_ERR_INDIVISIBLE", "TP_ERR_RANK", "TP_ERR_DTYPE",
          "TP_ERR_ALIGN", "TP_ERR_WORKSPACE", "TP_ERR_KV", "TP_ERR_ALIAS", "TP_ERR_HIP"]

EXPORTS = ["tp_shard_plan", "tp_linear_workspace_bytes", "tp_column_linear", "tp_swiglu",
           "tp_row_linear_partial", "tp_partial_sum", "tp_row_linear_partial_bf16", "tp_partial_sum_bf16",
           "tp_attention_workspace_bytes", "tp_decode_attention", "tp_prefill_attention",
           "tp_moe_workspace_bytes", "tp_moe_shard_forward", "tp_layer_workspace_bytes", "tp_layer_shard_forward",
           "tp_layer_shard_forward_static", "tp_hbm_stream_read", "tp_status_name", "tp_last_error"]


class tp_model_desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int64), ("intermediate", ctypes.c_int64),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("seq_len", ctypes.c_int64), ("batch", ctypes.c_int64),
                ("bytes_per_elem", ctypes.c_int32), ("eps", ctypes.c_float)]


class tp_rank_plan(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("q_head_begin", ctypes.c_int32), ("q_heads", ctypes.c_int32),
                ("kv_head_begin", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("inter_begin", ctypes.c_int64), ("inter_cols", ctypes.c_int64),
                ("qkv_cols", ctypes.c_int64), ("o_rows", ctypes.c_int64), ("weight_elems", ctypes.c_int64),
                ("kv_elems_per_seq_all_layers", ctypes.c_int64), ("kv_bytes_rank", ctypes.c_int64)]


class tp_rank_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down")]


class tp_kv_view(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("capacity", ctypes.c_int64),
                ("kv_len", ctypes.c_int64), ("new_tokens", ctypes.c_int64)]


class tp_moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("norm", "w_router", "w_gate", "w_up", "w_down")]


_P, _I64, _I32, _F, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "tp_shard_plan": (_I32, [ctypes.POINTER(tp_model_desc), _I32, _I32, ctypes.POINTER(tp_rank_plan)]),
    "tp_linear_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I32, _I32]),
    "tp_column_linear": (_I32, [_P, _P, _P, _P, _F, _P, _I64, _I64, _I64, _I32, _P, _SZ, _P]),
    "tp_swiglu": (_I32, [_P, _P, _P, _I64, _I64, _I32, _P]),
    "tp_row_linear_partial": (_I32, [_P, _P, _P, _I64, _I64, _I64, _I32, _P, _SZ, _P]),
    "tp_partial_sum": (_I32, [ctypes.POINTER(_P), _I32, _P, _P, _I64, _I64, _I32, _P]),
    "tp_row_linear_partial_bf16": (_I32, [_P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]),
    "tp_partial_sum_bf16": (_I32, [ctypes.POINTER(_P), _I32, _P, _P, _I64, _I64, _I32, _P]),
    "tp_attention_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I64]),
    "tp_decode_attention": (_I32, [_P, _P, _P, _P, _I64, _I32, _I32, _I32, _I64, _I64, _I32, _P, _SZ, _P]),
    "tp_prefill_attention": (_I32, [_P, _P, _P, _P, _I64, _I64, _I32, _I32, _I32, _I64, _I64, _I32, _P]),
    "tp_moe_workspace_bytes": (_SZ, [_I64, _I64, _I32, _I32, _I64, _I32]),
    "tp_moe_shard_forward": (_I32, [ctypes.POINTER(tp_moe_weights), _P, _P, _P, _P, _I64, _I64, _I32, _I32, _I64,
                                    _F, _P, _SZ, _P]),
    "tp_layer_workspace_bytes": (_SZ, [ctypes.POINTER(tp_model_desc), ctypes.POINTER(tp_rank_plan), _I32,
                                       _I64, _I32]),
    "tp_layer_shard_forward": (_I32, [ctypes.POINTER(tp_model_desc), ctypes.POINTER(tp_rank_plan), _I32,
                                      ctypes.POINTER(tp_rank_weights), _P, ctypes.POINTER(tp_kv_view), _P, _I64,
                                      _I32, _P, _SZ, _P]),
    "tp_layer_shard_forward_static": (_I32, [ctypes.POINTER(tp_model_desc), ctypes.POINTER(tp_rank_plan), _I32,
                                             ctypes.POINTER(tp_rank_weights), _P, ctypes.POINTER(tp_kv_view), _P,
                                             _I64, _I32, _P]),
    "tp_hbm_stream_read": (_I32, [_P, _SZ, _P, ctypes.c_uint32, _P]),
    "tp_status_name": (ctypes.c_char_p, [_I32]),
    "tp_last_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class TPError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = STATUS[status] if 0 <= status < len(STATUS) else str(status)
        super().__init__(f"{self.status}: {message}")


def _check(status: int) -> None:
    if status != 0:
        raise TPError(status, lib.tp_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TP_BF16
    if t.dtype == torch.float32:
        return TP_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def workspace(nbytes: int, device=None) -> torch.Tensor:
    """Zero-filled device scratch of at least nbytes (the workspace contract asks zeros once)."""
    return torch.zeros(max(int(nbytes), 256) + 256, dtype=torch.uint8, device=device or "cuda")


def _ws(ws: Optional[torch.Tensor]):
    if ws is None:
        return None, 0
    p = ws.data_ptr()
    aligned = (p + 255) // 256 * 256
    return aligned, ws.numel() * ws.element_size() - (aligned - p)


# ------------------------------------------------------------------ planner

def make_desc(hidden: int, intermediate: int = 0, n_q_heads: int = 0, n_kv_heads: int = 0, head_dim: int = 0,
              n_layers: int = 1, seq_len: int = 0, batch: int = 1, bytes_per_elem: int = 2,
              eps: float = 1e-5) -> tp_model_desc:
    return tp_model_desc(hidden, intermediate, n_q_heads, n_kv_heads, head_dim, n_layers, seq_len, batch,
                         bytes_per_elem, eps)


def tp_shard_plan(desc: tp_model_desc, t: int, rank: int) -> tp_rank_plan:
    out = tp_rank_plan()
    _check(lib.tp_shard_plan(ctypes.byref(desc), t, rank, ctypes.byref(out)))
    return out


def plan_dict(p: tp_rank_plan) -> Dict[str, int]:
    return {name: getattr(p, name) for name, _ in tp_rank_plan._fields_}


# ------------------------------------------------------------------ projections

def tp_linear_workspace_bytes(m: int, k: int, n: int, dtype: int, flags: int = 0) -> int:
    return lib.tp_linear_workspace_bytes(m, k, n, dtype, flags)


def tp_column_linear(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor, w_up: Optional[torch.Tensor] = None,
                     gamma: Optional[torch.Tensor] = None, eps: float = 1e-5, ws: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """y[m, n] = (u @ w^T) or silu(u @ w^T) * (u @ w_up^T); u = RMSNorm(x; gamma) if gamma given."""
    m, k = x.shape
    n = w.shape[0]
    dt = _dtype_code(x)
    if ws is None:
        flags = (TP_LINEAR_SWIGLU if w_up is not None else 0) | (TP_LINEAR_NORM if gamma is not None else 0)
        ws = workspace(tp_linear_workspace_bytes(m, k, n, dt, flags), x.device)
    wp, wn = _ws(ws)
    _check(lib.tp_column_linear(_ptr(x), _ptr(w), _ptr(w_up), _ptr(gamma), eps, _ptr(y), m, k, n, dt, wp, wn,
                                _stream(stream)))
    return y


def tp_swiglu(gate: torch.Tensor, up: torch.Tensor, out: torch.Tensor, stream=None) -> torch.Tensor:
    m, n = gate.shape
    _check(lib.tp_swiglu(_ptr(gate), _ptr(up), _ptr(out), m, n, _dtype_code(gate), _stream(stream)))
    return out


def tp_row_linear_partial(a: torch.Tensor, w: torch.Tensor, partial: torch.Tensor,
                          ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """partial[m, n] (float32) = a @ w^T."""
    m, k = a.shape
    n = w.shape[0]
    dt = _dtype_code(a)
    if ws is None:
        ws = workspace(tp_linear_workspace_bytes(m, k, n, dt, 0), a.device)
    wp, wn = _ws(ws)
    _check(lib.tp_row_linear_partial(_ptr(a), _ptr(w), _ptr(partial), m, k, n, dt, wp, wn, _stream(stream)))
    return partial


def tp_partial_sum(partials: Sequence[torch.Tensor], out: torch.Tensor, residual: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """out = sum of the partials in rank order (+ residual)."""
    t = len(partials)
    m, n = out.shape
    arr = (ctypes.c_void_p * max(t, 1))(*[_ptr(p) for p in partials])
    _check(lib.tp_partial_sum(arr, t, _ptr(residual), _ptr(out), m, n, _dtype_code(out), _stream(stream)))
    return out


def tp_row_linear_partial_bf16(a: torch.Tensor, w: torch.Tensor, partial: torch.Tensor,
                               ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """partial[m, n] = bf16(a @ w^T); a, w, partial bf16."""
    m, k = a.shape
    n = w.shape[0]
    if ws is None:
        ws = workspace(tp_linear_workspace_bytes(m, k, n, TP_BF16), a.device)
    wp, wn = _ws(ws)
    _check(lib.tp_row_linear_partial_bf16(_ptr(a), _ptr(w), _ptr(partial), m, k, n, wp, wn, _stream(stream)))
    return partial


def tp_partial_sum_bf16(partials: Sequence[torch.Tensor], out: torch.Tensor, residual: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """out = sum of t bf16 partials (float32 arithmetic, rank order) (+ residual)."""
    t = len(partials)
    m, n = out.shape
    arr = (ctypes.c_void_p * max(t, 1))(*[_ptr(p) for p in partials])
    _check(lib.tp_partial_sum_bf16(arr, t, _ptr(residual), _ptr(out), m, n, _dtype_code(out), _stream(stream)))
    return out


# ------------------------------------------------------------------ attention and layer

def tp_attention_workspace_bytes(batch: int, q_heads: int, kv_heads: int, head_dim: int, kv_len: int) -> int:
    return lib.tp_attention_workspace_bytes(batch, q_heads, kv_heads, head_dim, kv_len)


def tp_decode_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, kv_len: int,
                        q_heads: int, ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q, out [B, q_heads*d]; k, v [B, kv_heads, capacity, d]."""
    B, kv_heads, cap, d = k.shape
    if ws is None:
        ws = workspace(tp_attention_workspace_bytes(B, q_heads, kv_heads, d, kv_len), q.device)
    wp, wn = _ws(ws)
    _check(lib.tp_decode_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, q_heads, kv_heads, d, cap, kv_len,
                                   _dtype_code(q), wp, wn, _stream(stream)))
    return out


def tp_prefill_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, kv_len: int,
                         q_heads: int, stream=None) -> torch.Tensor:
    """q, out [B, S, q_heads*d]; k, v [B, kv_heads, capacity, d]; tokens at kv_len-S .. kv_len-1."""
    B, kv_heads, cap, d = k.shape
    S = q.shape[1]
    _check(lib.tp_prefill_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S, q_heads, kv_heads, d, cap, kv_len,
                                    _dtype_code(q), _stream(stream)))
    return out


def tp_moe_workspace_bytes(m: int, hidden: int, n_experts: int, top_k: int, inter_cols: int,
                           has_norm: bool = True) -> int:
    return lib.tp_moe_workspace_bytes(m, hidden, n_experts, top_k, inter_cols, int(bool(has_norm)))


def tp_moe_shard_forward(weights: Dict[str, torch.Tensor], x: torch.Tensor, partial: torch.Tensor, n_experts: int,
                         top_k: int, inter_cols: int, eps: float = 1e-5, gates: Optional[torch.Tensor] = None,
                         logits: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """One rank's MoE FFN: weights {"norm", "w_router", "w_gate", "w_up", "w_down"} (experts stacked)."""
    m, H = x.shape
    w = tp_moe_weights(*[_ptr(weights.get(n)) for n in ("norm", "w_router", "w_gate", "w_up", "w_down")])
    if ws is None:
        ws = workspace(tp_moe_workspace_bytes(m, H, n_experts, top_k, inter_cols, weights.get("norm") is not None),
                       x.device)
    wp, wn = _ws(ws)
    _check(lib.tp_moe_shard_forward(ctypes.byref(w), _ptr(x), _ptr(partial), _ptr(gates), _ptr(logits), m, H,
                                    n_experts, top_k, inter_cols, eps, wp, wn, _stream(stream)))
    return partial


def tp_layer_workspace_bytes(desc: tp_model_desc, plan: tp_rank_plan, stage: int, m: int, dtype: int) -> int:
    return lib.tp_layer_workspace_bytes(ctypes.byref(desc), ctypes.byref(plan), stage, m, dtype)


def tp_layer_shard_forward(desc: tp_model_desc, plan: tp_rank_plan, stage: int, weights: Dict[str, torch.Tensor],
                           inp: torch.Tensor, partial: torch.Tensor, kv: Optional[Dict] = None,
                           ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One rank's ATTN or MLP block; ``kv`` = {"k", "v", "kv_len"[, "new_tokens"]} for ATTN.

    inp [m, H]: m sequences of one new token, or with ``new_tokens`` = S > 1,
    m / S sequences of S new tokens each, rows sequence-major."""
    m = inp.shape[0]
    dt = _dtype_code(inp)
    w = tp_rank_weights(*[_ptr(weights.get(n)) for n in
                          ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down")])
    kvv = None
    if kv is not None:
        kvv = tp_kv_view(_ptr(kv["k"]), _ptr(kv["v"]), kv["k"].shape[2], kv["kv_len"], kv.get("new_tokens", 1))
    if ws is None:
        ws = workspace(tp_layer_workspace_bytes(desc, plan, stage, m, dt), inp.device)
    wp, wn = _ws(ws)
    _check(lib.tp_layer_shard_forward(ctypes.byref(desc), ctypes.byref(plan), stage, ctypes.byref(w), _ptr(inp),
                                      ctypes.byref(kvv) if kvv is not None else None, _ptr(partial), m, dt, wp, wn,
                                      _stream(stream)))
    return partial


def tp_layer_shard_forward_static(desc: tp_model_desc, plan: tp_rank_plan, stage: int,
                                  weights: Dict[str, torch.Tensor], inp: torch.Tensor, partial: torch.Tensor,
                                  kv: Optional[Dict] = None, stream=None) -> torch.Tensor:
    """tp_layer_shard_forward with the library's per-GPU static scratch in place of a workspace."""
    m = inp.shape[0]
    w = tp_rank_weights(*[_ptr(weights.get(n)) for n in
                          ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down")])
    kvv = None
    if kv is not None:
        kvv = tp_kv_view(_ptr(kv["k"]), _ptr(kv["v"]), kv["k"].shape[2], kv["kv_len"], kv.get("new_tokens", 1))
    _check(lib.tp_layer_shard_forward_static(ctypes.byref(desc), ctypes.byref(plan), stage, ctypes.byref(w),
                                             _ptr(inp), ctypes.byref(kvv) if kvv is not None else None,
                                             _ptr(partial), m, _dtype_code(inp), _stream(stream)))
    return partial


# ------------------------------------------------------------------ measurement helper

def tp_hbm_stream_read(buf: torch.Tensor, flag: torch.Tensor, never: int = 0x9E3779B9, stream=None) -> None:
    """Read every byte of buf once (the practical HBM read rate); flag: a 4-byte device word."""
    _check(lib.tp_hbm_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(flag), never,
                                  _stream(stream)))
