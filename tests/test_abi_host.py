"""The C ABI on the host (no GPU): symbols, planner against the oracle, validation.

Every call here fails validation before anything is enqueued, so fake but
aligned pointers are safe: the library never dereferences them.
"""
import ctypes
import itertools
import os
import re

import pytest

import megatron_tensor_transformer_amd as tp
from oracle import plan as oplan

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "tp_shard.h")
A = 0x7f0000000000          # fake, 256-byte aligned address
MB = 1 << 20


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(tp_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_six_entry_points():
    names = declared_functions()
    for n in ["tp_shard_plan", "tp_column_linear", "tp_swiglu", "tp_row_linear_partial", "tp_partial_sum",
              "tp_layer_shard_forward"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(tp.lib, n), n
    assert sorted(tp.EXPORTS) == names


def test_one_hip_runtime_mapped():
    maps = open("/proc/self/maps").read()
    paths = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(paths) == 1, paths


def test_status_names():
    for i, name in enumerate(tp.STATUS):
        assert tp.lib.tp_status_name(i).decode() == name


def desc_of(d: oplan.ModelDesc):
    return tp.make_desc(d.hidden, d.intermediate, d.n_q_heads, d.n_kv_heads, d.head_dim, d.n_layers, d.seq_len,
                        d.batch, d.bytes_per_elem)


def test_plan_matches_oracle():
    shapes = [
        oplan.ModelDesc(hidden=8192, intermediate=28672, n_q_heads=64, n_kv_heads=8, head_dim=128, n_layers=80,
                        seq_len=8192, batch=16, bytes_per_elem=2),
        oplan.ModelDesc(hidden=4096, intermediate=14336, n_q_heads=32, n_kv_heads=8, head_dim=128, n_layers=32,
                        seq_len=4096, batch=4),
        oplan.ModelDesc(hidden=256, intermediate=1024),
        oplan.ModelDesc(hidden=96, intermediate=48, n_q_heads=12, n_kv_heads=6, head_dim=8, seq_len=7, batch=3),
        oplan.ModelDesc(hidden=4096, intermediate=14336, n_q_heads=32, n_kv_heads=2, head_dim=128, n_layers=4,
                        seq_len=64, batch=2, bytes_per_elem=2),             # t = 4, 8: kv heads replicated
        oplan.ModelDesc(hidden=64, intermediate=64, n_q_heads=8, n_kv_heads=1, head_dim=8, seq_len=5, batch=1),
    ]
    for d, t in itertools.product(shapes, range(1, 9)):
        for r in range(t):
            try:
                ref = oplan.rank_plan(d, t, r)
            except oplan.PlanError as e:
                with pytest.raises(tp.TPError) as ei:
                    tp.tp_shard_plan(desc_of(d), t, r)
                assert ei.value.status == "TP_ERR_" + e.kind
                continue
            got = tp.plan_dict(tp.tp_shard_plan(desc_of(d), t, r))
            for k, v in ref.items():
                assert got[k] == v, (d, t, r, k)


def test_plan_kv_worked_example():
    d = tp.make_desc(8192, 28672, 64, 8, 128, n_layers=80, seq_len=8192, batch=16, bytes_per_elem=2)
    p = tp.tp_shard_plan(d, 4, 0)
    assert p.kv_elems_per_seq_all_layers == 1_342_177_280
    assert p.kv_bytes_rank == 10 * (1 << 30)


@pytest.mark.parametrize("t,rank,kind", [(0, 0, "TP_ERR_RANK"), (9, 0, "TP_ERR_RANK"), (4, 4, "TP_ERR_RANK"),
                                         (3, 0, "TP_ERR_INDIVISIBLE")])
def test_plan_errors(t, rank, kind):
    d = tp.make_desc(8192, 28672, 64, 8, 128)
    with pytest.raises(tp.TPError) as e:
        tp.tp_shard_plan(d, t, rank)
    assert e.value.status == kind
    assert tp.lib.tp_last_error().decode()


def test_plan_null():
    out = tp.tp_rank_plan()
    assert tp.lib.tp_shard_plan(None, 1, 0, ctypes.byref(out)) == 1


def rejected(status: int) -> str:
    """Name of a status that must be a validation failure (nothing enqueued)."""
    name = tp.STATUS[status]
    assert name not in ("TP_OK", "TP_ERR_HIP"), "a call with fake pointers passed validation"
    return name


def col(x=A, w=A + 64 * MB, w_up=None, gamma=None, eps=1e-5, y=A + 128 * MB, m=4, k=256, n=512, dt=tp.TP_BF16,
        ws=None, wsn=0):
    return rejected(tp.lib.tp_column_linear(x, w, w_up, gamma, eps, y, m, k, n, dt, ws, wsn, None))


def test_column_linear_validation():
    assert col(x=None) == "TP_ERR_NULL"
    assert col(w=None) == "TP_ERR_NULL"
    assert col(y=None) == "TP_ERR_NULL"
    assert col(x=A + 8) == "TP_ERR_ALIGN"
    assert col(w_up=A + 200 * MB + 4) == "TP_ERR_ALIGN"
    assert col(m=0) == "TP_ERR_SHAPE"
    assert col(n=-1) == "TP_ERR_SHAPE"
    assert col(k=1 << 31) == "TP_ERR_SHAPE"
    assert col(k=260) == "TP_ERR_ALIGN"                      # bf16 needs k % 8 == 0
    assert col(dt=7) == "TP_ERR_DTYPE"
    assert col(y=A + 1024) == "TP_ERR_ALIAS"                 # y inside x
    assert col(eps=-1.0) == "TP_ERR_SHAPE"
    # a split-K shape needs a workspace
    need = tp.tp_linear_workspace_bytes(16, 8192, 1280, tp.TP_BF16, 0)
    assert need > 0
    assert col(m=16, k=8192, n=1280, ws=None) == "TP_ERR_WORKSPACE"
    assert col(m=16, k=8192, n=1280, ws=A + 512 * MB, wsn=need - 1) == "TP_ERR_WORKSPACE"
    assert col(m=16, k=8192, n=1280, ws=A + 512 * MB + 16, wsn=need) == "TP_ERR_WORKSPACE"
    assert col(m=16, k=8192, n=1280, y=A + 600 * MB, ws=A + 600 * MB, wsn=need) == "TP_ERR_ALIAS"


def test_col_k_f32_multiple_of_4():
    assert col(k=258, dt=tp.TP_F32) == "TP_ERR_ALIGN"


def test_row_linear_validation():
    f = lambda **kw: rejected(tp.lib.tp_row_linear_partial(kw.get("a", A), kw.get("w", A + 64 * MB),
                                                            kw.get("p", A + 128 * MB), kw.get("m", 4),
                                                            kw.get("k", 512), kw.get("n", 256),
                                                            kw.get("dt", tp.TP_BF16), kw.get("ws"), kw.get("wsn", 0),
                                                            None))
    assert f(a=None) == "TP_ERR_NULL"
    assert f(p=A + 16 * MB + 8) == "TP_ERR_ALIGN"
    assert f(k=0) == "TP_ERR_SHAPE"
    assert f(k=12) == "TP_ERR_ALIGN"
    assert f(p=A + 64 * MB + 256) == "TP_ERR_ALIAS"
    assert f(dt=3) == "TP_ERR_DTYPE"


def test_swiglu_validation():
    f = lambda g=A, u=A + MB, o=A + 2 * MB, m=4, n=64, dt=tp.TP_BF16: rejected(
        tp.lib.tp_swiglu(g, u, o, m, n, dt, None))
    assert f(g=None) == "TP_ERR_NULL"
    assert f(o=A + 16) == "TP_ERR_ALIAS"            # partial overlap with gate
    assert f(m=0) == "TP_ERR_SHAPE"
    assert f(u=A + MB + 2) == "TP_ERR_ALIGN"


def test_partial_sum_validation():
    def f(ptrs, t, res=None, out=A + 100 * MB, m=4, n=64, dt=tp.TP_F32):
        arr = (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)
        return rejected(tp.lib.tp_partial_sum(arr, t, res, out, m, n, dt, None))
    ptrs = [A + i * MB for i in range(8)]
    assert f(ptrs, 0) == "TP_ERR_RANK"
    assert f(ptrs, 9) == "TP_ERR_RANK"
    assert f([A, None], 2) == "TP_ERR_NULL"
    assert f([A, A + 4], 2) == "TP_ERR_ALIGN"
    assert f(ptrs, 4, out=A + 2 * MB) == "TP_ERR_ALIAS"
    assert f(ptrs, 4, res=A + 100 * MB + 16) == "TP_ERR_ALIAS"
    assert f(ptrs, 4, m=-3) == "TP_ERR_SHAPE"
    assert f(ptrs, 4, dt=9) == "TP_ERR_DTYPE"
    assert rejected(tp.lib.tp_partial_sum(None, 2, None, A, 4, 4, 0, None)) == "TP_ERR_NULL"


def test_bf16_partial_validation():
    def row(a=A, w=A + 64 * MB, part=A + 128 * MB, m=4, k=256, n=512, ws=None, wsn=0):
        return rejected(tp.lib.tp_row_linear_partial_bf16(a, w, part, m, k, n, ws, wsn, None))
    assert row(a=None) == "TP_ERR_NULL"
    assert row(k=260) == "TP_ERR_ALIGN"
    assert row(part=A + 16) == "TP_ERR_ALIAS"
    assert row(m=0) == "TP_ERR_SHAPE"

    def f(ptrs, t, res=None, out=A + 100 * MB, m=4, n=64, dt=tp.TP_BF16):
        arr = (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)
        return rejected(tp.lib.tp_partial_sum_bf16(arr, t, res, out, m, n, dt, None))
    ptrs = [A + i * MB for i in range(8)]
    assert f(ptrs, 0) == "TP_ERR_RANK"
    assert f([A, None], 2) == "TP_ERR_NULL"
    assert f(ptrs, 4, out=A + 2 * MB + 256) == "TP_ERR_ALIAS"
    assert f(ptrs, 4, dt=7) == "TP_ERR_DTYPE"


def test_moe_validation():
    w = tp.tp_moe_weights(A, A + 64 * MB, A + 128 * MB, A + 1024 * MB, A + 2048 * MB)
    need = tp.tp_moe_workspace_bytes(16, 4096, 8, 2, 7168, True)
    assert need > 16 * 8 * 7168 * 2

    def f(weights=w, x=A + 3000 * MB, part=A + 3100 * MB, g=None, lg=None, m=16, H=4096, E=8, k=2, cols=7168,
          eps=1e-5, ws=A + 3200 * MB, wsn=None):
        return rejected(tp.lib.tp_moe_shard_forward(ctypes.byref(weights) if weights is not None else None, x, part,
                                                    g, lg, m, H, E, k, cols, eps, ws, need if wsn is None else wsn,
                                                    None))
    assert f(weights=None) == "TP_ERR_NULL"
    assert f(x=None) == "TP_ERR_NULL"
    assert f(E=65) == "TP_ERR_SHAPE"
    assert f(k=9) == "TP_ERR_SHAPE"
    assert f(k=0) == "TP_ERR_SHAPE"
    assert f(cols=7170) == "TP_ERR_ALIGN"
    assert f(part=A + 3000 * MB + 256) == "TP_ERR_ALIAS"
    assert f(wsn=need - 256) == "TP_ERR_WORKSPACE"
    assert f(g=A + 5) == "TP_ERR_ALIGN"
    assert tp.tp_moe_workspace_bytes(16, 4096, 0, 1, 7168, True) == 0
    assert tp.tp_moe_workspace_bytes(16, 4096, 8, 9, 7168, True) == 0
    # above 64 tokens each expert runs over its own tokens: activations for m * top_k rows, and the
    # top_k slot partials
    big = tp.tp_moe_workspace_bytes(4096, 4096, 8, 2, 7168, True)
    assert big >= 4096 * 2 * 7168 * 2 + 2 * 4096 * 4096 * 4
    assert big < 4096 * 8 * 7168 * 2 + 2 * 4096 * 4096 * 4 + (64 << 20)


def attn(q=A, k=A + 64 * MB, v=A + 128 * MB, out=A + 192 * MB, B=16, qh=8, kvh=1, d=128, cap=8192, L=8192,
         dt=tp.TP_BF16, ws=None, wsn=0):
    return rejected(tp.lib.tp_decode_attention(q, k, v, out, B, qh, kvh, d, cap, L, dt, ws, wsn, None))


def test_attention_validation():
    assert attn(dt=tp.TP_F32) == "TP_ERR_DTYPE"
    assert attn(q=None) == "TP_ERR_NULL"
    assert attn(L=0) == "TP_ERR_KV"
    assert attn(L=8193) == "TP_ERR_KV"
    assert attn(d=96) == "TP_ERR_SHAPE"
    assert attn(qh=24, kvh=8) == "TP_ERR_SHAPE"      # 3 q heads per kv head
    assert attn(qh=9, kvh=2) == "TP_ERR_INDIVISIBLE"
    assert attn(out=A + 64 * MB + 256) == "TP_ERR_ALIAS"
    assert attn(ws=None) == "TP_ERR_WORKSPACE"       # 8192 keys split over workgroups
    assert tp.tp_attention_workspace_bytes(16, 8, 1, 128, 8192) > 0


def prefill(q=A, k=A + 64 * MB, v=A + 128 * MB, out=A + 192 * MB, B=2, S=2048, qh=8, kvh=1, d=128, cap=2048,
            L=2048, dt=tp.TP_BF16):
    return rejected(tp.lib.tp_prefill_attention(q, k, v, out, B, S, qh, kvh, d, cap, L, dt, None))


def test_prefill_attention_validation():
    assert prefill(dt=tp.TP_F32) == "TP_ERR_DTYPE"
    assert prefill(v=None) == "TP_ERR_NULL"
    assert prefill(out=A + 192 * MB + 4) == "TP_ERR_ALIGN"
    assert prefill(S=0) == "TP_ERR_KV"
    assert prefill(S=2049) == "TP_ERR_KV"            # more new tokens than keys
    assert prefill(L=2049) == "TP_ERR_KV"            # beyond the cache
    assert prefill(d=96) == "TP_ERR_SHAPE"
    assert prefill(qh=32, kvh=1) == "TP_ERR_SHAPE"   # 32 q heads per kv head
    assert prefill(qh=9, kvh=2) == "TP_ERR_INDIVISIBLE"
    assert prefill(B=70000) == "TP_ERR_SHAPE"
    assert prefill(out=A + 64 * MB + 256) == "TP_ERR_ALIAS"
    assert prefill(out=A + 4 * MB) == "TP_ERR_ALIAS"  # inside q


def test_layer_validation():
    d = tp.make_desc(8192, 28672, 64, 8, 128, seq_len=8192, batch=16)
    p = tp.tp_shard_plan(d, 8, 3)
    w = tp.tp_rank_weights(*[A + i * 256 * MB for i in range(7)])
    kv = tp.tp_kv_view(A + 4096 * MB, A + 5120 * MB, 8192, 8192, 1)

    def f(stage=tp.TP_STAGE_MLP, plan=p, weights=w, inp=A + 3000 * MB, kvv=kv, part=A + 3100 * MB, m=16,
          dt=tp.TP_BF16, ws=None, wsn=0):
        return rejected(tp.lib.tp_layer_shard_forward(ctypes.byref(d), ctypes.byref(plan), stage,
                                                      ctypes.byref(weights) if weights is not None else None,
                                                      inp, ctypes.byref(kvv) if kvv is not None else None,
                                                      part, m, dt, ws, wsn, None))
    bad = tp.tp_shard_plan(d, 8, 3)
    bad.inter_begin += 1
    assert f(plan=bad) == "TP_ERR_SHAPE"
    assert f(weights=None) == "TP_ERR_NULL"
    assert f(stage=tp.TP_STAGE_ATTN, kvv=None) == "TP_ERR_NULL"
    assert f(stage=tp.TP_STAGE_ATTN, dt=tp.TP_F32) == "TP_ERR_DTYPE"
    assert f(stage=tp.TP_STAGE_ATTN, kvv=tp.tp_kv_view(A + 4096 * MB, A + 5120 * MB, 8192, 0, 1)) == "TP_ERR_KV"
    kvp = lambda kv_len, new: tp.tp_kv_view(A + 4096 * MB, A + 5120 * MB, 8192, kv_len, new)
    assert f(stage=tp.TP_STAGE_ATTN, kvv=kvp(8192, -1)) == "TP_ERR_SHAPE"     # negative block
    assert f(stage=tp.TP_STAGE_ATTN, kvv=kvp(8192, 3)) == "TP_ERR_SHAPE"      # 16 rows are not 3-token blocks
    assert f(stage=tp.TP_STAGE_ATTN, kvv=kvp(7, 8)) == "TP_ERR_KV"            # block longer than kv_len
    assert f(inp=None) == "TP_ERR_NULL"
    assert f(part=A + 3000 * MB + 64) == "TP_ERR_ALIAS"
    assert f(ws=None) in ("TP_ERR_WORKSPACE",)
    assert f(stage=5) == "TP_ERR_SHAPE"
    need_attn = tp.tp_layer_workspace_bytes(d, p, tp.TP_STAGE_ATTN, 16, tp.TP_BF16)
    need_mlp = tp.tp_layer_workspace_bytes(d, p, tp.TP_STAGE_MLP, 16, tp.TP_BF16)
    assert need_attn > 16 * 1024 * 2 * 2 and need_mlp > 16 * 3584 * 2
    assert f(ws=A + 6000 * MB, wsn=need_mlp - 1) == "TP_ERR_WORKSPACE"
    # m rows of a 2048-token block: the [q | k | v] rows and the attention output fit the workspace
    need_pre = tp.tp_layer_workspace_bytes(d, p, tp.TP_STAGE_ATTN, 4096, tp.TP_BF16)
    assert need_pre >= 4096 * (p.qkv_cols + p.o_rows) * 2
    assert f(stage=tp.TP_STAGE_ATTN, kvv=kvp(8192, 2048), m=4096, ws=A + 6000 * MB,
             wsn=4096 * p.qkv_cols * 2) == "TP_ERR_WORKSPACE"


def test_workspace_sizes_are_zero_for_bad_args():
    assert tp.tp_linear_workspace_bytes(0, 8, 8, tp.TP_BF16, 0) == 0
    assert tp.tp_attention_workspace_bytes(1, 3, 2, 128, 10) == 0


def test_linear_workspace_follows_the_k_split_rule():
    """Decode projections whose row tiles fill the chip keep all of K in one workgroup and need no
    workspace; narrower ones, or K beyond one workgroup's reach, split K and need room for the slices."""
    BF = tp.TP_BF16
    for m, k, n in [(16, 3584, 4096),     # Llama-3-8B down (t=4): 256 tiles of 16 rows
                    (16, 2048, 8192),     # 70B W_o (t=4): 256 tiles of 32 rows
                    (16, 1024, 8192)]:    # 70B W_o (t=8)
        assert tp.tp_linear_workspace_bytes(m, k, n, BF, 0) == 0, (m, k, n)
    for m, k, n in [(16, 8192, 2560),     # 70B QKV (t=4): tiles of 10 rows would be too short
                    (16, 8192, 1280),     # 70B QKV (t=8)
                    (16, 8200, 8192),     # K past one workgroup's 8192
                    (16, 57344, 4096)]:   # the stacked Mixtral down projection
        assert tp.tp_linear_workspace_bytes(m, k, n, BF, 0) > 0, (m, k, n)


def test_hbm_stream_read_validation():
    f = tp.lib.tp_hbm_stream_read
    assert tp.STATUS[f(None, 16, 4096, 0, None)] == "TP_ERR_NULL"
    assert tp.STATUS[f(4096, 16, None, 0, None)] == "TP_ERR_NULL"
    assert tp.STATUS[f(4097, 16, 8192, 0, None)] == "TP_ERR_ALIGN"
    assert tp.STATUS[f(4096, 0, 8192, 0, None)] == "TP_ERR_SHAPE"
    assert tp.STATUS[f(4096, 24, 8192, 0, None)] == "TP_ERR_SHAPE"
    assert tp.STATUS[f(4096, 64, 4112, 0, None)] == "TP_ERR_ALIAS"


def test_static_entry_refuses_calls_beyond_its_scratch():
    """A 2 x 2048-token prefill block of the 70B layer at t=8 needs more than the static scratch; the
    allocation-free entry point refuses it before any HIP call."""
    d = tp.make_desc(8192, 28672, 64, 8, 128, n_layers=1, seq_len=2048, batch=2)
    p = tp.tp_shard_plan(d, 8, 0)
    assert tp.tp_layer_workspace_bytes(d, p, tp.TP_STAGE_ATTN, 4096, tp.TP_BF16) > 16 * MB
    w = tp.tp_rank_weights(A, A, A, A, A, A, A)
    kv = tp.tp_kv_view(A + 4096 * MB, A + 5000 * MB, 2048, 2048, 2048)
    st = tp.lib.tp_layer_shard_forward_static(ctypes.byref(d), ctypes.byref(p), tp.TP_STAGE_ATTN, ctypes.byref(w),
                                              A + 64 * MB, ctypes.byref(kv), A + 512 * MB, 4096, tp.TP_BF16, None)
    assert tp.STATUS[st] == "TP_ERR_WORKSPACE"
    assert "static scratch" in tp.lib.tp_last_error().decode()
