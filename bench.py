"""Throughput of one GPU's tensor-parallel layer shards on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload mlp_decode|attn_proj|mlp_prefill|layer_decode] [--tokens M] [--no-cpu]

Workloads (synthetic, seeded inputs already in HBM; every rank shard of the
tensor-parallel group runs on the one device, then the on-device sum of the t
partials):

  mlp_decode (default)  Llama-3-8B-shaped MLP block, hidden 4096, intermediate
                        14336, t=4, 16 tokens, RMSNorm in front: per rank fused
                        RMSNorm + gate/up + SwiGLU, then the down row-partial.
  attn_proj             70B-shaped attention projections, hidden 8192, 64 q / 8
                        kv heads of 128, t=4, 16 tokens: per rank the QKV column
                        projection and the W_o row-partial.
  mlp_prefill           70B-shaped MLP block, hidden 8192, intermediate 28672,
                        t=4, 4096 tokens (MFMA GEMMs); metric in TFLOP/s.
  layer_decode          70B-shaped full layer, t=8, batch 16, KV cache of 8192
                        tokens: per rank RMSNorm + QKV (+ KV append), GQA decode
                        attention, W_o partial; sum + residual; RMSNorm +
                        gate/up + SwiGLU, down partial; sum + residual.

One step is one pass of that whole path; K steps are replayed from HIP graphs
and timed between two events. Prints one JSON line. ``value`` is the step's
throughput; ``roofline`` rates the dominant kernel by its algorithmic bytes
(or flops) over its average duration, from HIP events around back-to-back
launches on the stream it runs on; ``cpu_baseline`` times the float64 CPU
oracle on a bounded sample of the same workload.

``--calibrate-copy`` adds a plain 256 MiB device copy before the timed region;
hardware-counter runs use it to scale FETCH_SIZE / WRITE_SIZE to bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s & HBM GB/s (% peak); prefill TFLOP/s (% MFMA peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mlp_decode",
                    choices=["mlp_decode", "attn_proj", "mlp_prefill", "layer_decode", "attn_prefill",
                             "layer_prefill", "moe_decode"])
    ap.add_argument("--tokens", type=int, default=None, help="batch of the timed step (default: the workload's)")
    ap.add_argument("--copies", type=int, default=None, help="weight copies the steps rotate over")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true")
    return ap.parse_args()


class Ctx:
    """Handles shared by the workloads."""

    def __init__(self, args):
        import torch

        import megatron_tensor_transformer_amd as tp
        import workloads as W
        self.args, self.torch, self.tp, self.W = args, torch, tp, W

    def dev(self, a, dt="bf16"):
        torch = self.torch
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        return (t.to(torch.bfloat16) if dt == "bf16" else t).cuda()

    def phys(self, a):
        """A logical [in, out] weight as the row-major [out, in] matrix the kernels read."""
        return np.ascontiguousarray(np.asarray(a).T)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's shard: only --gpus 1 is supported (the t rank shards of a layer run "
              "one after another on the single device and their partials are summed there).", file=sys.stderr)
        sys.exit(2)
    ctx = Ctx(args)
    torch = ctx.torch
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    bench = {"mlp_decode": bench_mlp_decode, "attn_proj": bench_attn_proj, "mlp_prefill": bench_mlp_prefill,
             "layer_decode": bench_layer_decode, "attn_prefill": bench_attn_prefill,
             "layer_prefill": bench_layer_prefill, "moe_decode": bench_moe_decode}[args.workload]
    if args.calibrate_copy:
        calibrate_copy(torch)
    res = bench(ctx)
    res["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(res), flush=True)


# ----------------------------------------------------------------------------
# timing


_CYCLES_PER_MS = []


def gpu_hold(torch, ms=20.0):
    """Keep the stream busy for about ms so the host can queue work ahead of the timed region."""
    if not _CYCLES_PER_MS:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(100000)
        e0.record()
        torch.cuda._sleep(2000000)
        e1.record()
        torch.cuda.synchronize()
        _CYCLES_PER_MS.append(2000000 / max(e0.elapsed_time(e1), 1e-3))
    torch.cuda._sleep(int(min(ms, 200.0) * _CYCLES_PER_MS[0]))


def capture_steps(torch, step, n):
    """One HIP graph per weight copy: the step's launches, replayed without host overhead."""
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(n):
            step(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def time_steps(ctx, step, n_graphs):
    """Warm up eagerly, capture, warm up the graphs, then time ``steps`` replays. Returns total ms."""
    torch, args = ctx.torch, ctx.args
    log(f"[bench] warmup {args.warmup} eager steps")
    for i in range(max(args.warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    graphs = capture_steps(torch, step, n_graphs)
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} graph-replayed steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gpu_hold(torch)
    e0.record()
    for i in range(args.steps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def event_time_ms(torch, fn, n, reps=5):
    """Average ms per call of fn: n calls launched back to back between two HIP
    events on the stream they run on (torch's current stream, which the
    binding passes to every entry point), repeated ``reps`` times.

    A spin kernel first keeps the stream busy while every launch is queued, so
    the timed region never waits on the host. Returns (mean, median, min) over
    the repetitions of the per-call average."""
    per = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        gpu_hold(torch, 5.0 + 0.05 * n)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) / n)
    return float(np.mean(per)), float(np.median(per)), float(np.min(per))


def calibrate_copy(torch):
    """A plain device copy of COPY_BYTES (read once, written once), three times."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def projection_kernel(m, dtype="bf16", wide=False):
    """The kernel a projection of m tokens runs on (the library's dispatch rule); wide: one whose tiles
    fill the chip without splitting K (the 8B gate/up and down, the 70B W_o and t=8 MLP), which runs
    one K range per wave."""
    if dtype == "bf16" and m > 16:
        return "gemm_bf16_kernel (MFMA prefill GEMM)"
    if dtype == "bf16" and m >= 5:
        if wide:
            return "gemv_mfma_wide_kernel (matrix-core decode projection, one K range per wave)"
        return "gemv_mfma_kernel (matrix-core decode projection)"
    return "gemv_kernel (v_dot2 decode projection)"


def source_digest():
    """Digest of the kernel sources; hardware-counter figures are only reported while it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "megatron_tensor_transformer_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def counted_traffic(kernel_key):
    """HBM bytes per launch of a kernel from the committed counter summary, or None.

    The summary holds, per (kernel, workload) key, FETCH_SIZE and WRITE_SIZE
    in KiB per dispatch from two counter runs, and the same counters for the
    plain copy of known size that scales them to bytes. Figures taken for
    other kernel sources are not used."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#") or "=" not in line:
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_digest") != source_digest():
        return None
    try:
        fetch_scale = COPY_BYTES / (float(vals["copy.FETCH_SIZE_KiB"]) * 1024.0)
        write_scale = COPY_BYTES / (float(vals["copy.WRITE_SIZE_KiB"]) * 1024.0)
        fetch = float(vals[f"{kernel_key}.FETCH_SIZE_KiB"]) * 1024.0 * fetch_scale
        write = float(vals[f"{kernel_key}.WRITE_SIZE_KiB"]) * 1024.0 * write_scale
    except (KeyError, ValueError, ZeroDivisionError):
        return None
    return fetch + write


def roofline_hbm(kernel, key, nbytes, mean_ms, med_ms, min_ms):
    gbps = nbytes / (mean_ms * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS, "traffic": counted_traffic(key), "bytes_per_launch": nbytes,
            "us_mean": mean_ms * 1e3, "us_median": med_ms * 1e3, "us_min": min_ms * 1e3}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        th = [d.get("num_threads") for d in threadpool_info() if d.get("user_api") == "blas"]
        return max(th) if th else 1
    except Exception:                      # pragma: no cover
        return 1


def repeat_for(seconds, fn):
    """Run fn until about ``seconds`` have passed; returns (calls, elapsed)."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return n, el


def result(ctx, value, unit, ms_step, config, extra):
    args = ctx.args
    out = {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) activations and caches, N(0,0.02) weights)", "config": config}
    out.update(extra)
    return out


# ----------------------------------------------------------------------------
# workloads


def bench_mlp_decode(ctx):
    torch, tp, W, args = ctx.torch, ctx.tp, ctx.W, ctx.args
    wl = W.WORKLOADS[2]
    H, I, t = wl.hidden, wl.intermediate, wl.t
    M = args.tokens or 16
    copies_n = args.copies or 2
    log(f"[bench] drawing {wl.name}")
    inp = W.mlp_inputs(2, H, I, max(max(wl.tokens), M), "bf16", "ones")
    desc = tp.make_desc(H, I, eps=wl.eps)
    plans = [tp.tp_shard_plan(desc, t, r) for r in range(t)]
    I_r = plans[0].inter_cols
    gam = ctx.dev(inp["gamma"])
    copies = []
    for _ in range(copies_n):
        ranks = []
        for p in plans:
            b, n = p.inter_begin, p.inter_cols
            ranks.append({"mlp_norm": gam, "w_gate": ctx.dev(ctx.phys(inp["w_gate"][:, b:b + n])),
                          "w_up": ctx.dev(ctx.phys(inp["w_up"][:, b:b + n])),
                          "w_down": ctx.dev(ctx.phys(inp["w_down"][b:b + n]))})
        copies.append(ranks)
    ws = tp.workspace(max(tp.tp_layer_workspace_bytes(desc, p, tp.TP_STAGE_MLP, max(max(wl.tokens), M), tp.TP_BF16)
                          for p in plans))
    nlaunch = max(copies_n * t * 16, 64)

    # one rank's shard and its dominant kernel, at every batch size of the workload
    per_batch = {}
    for m in sorted(set(wl.tokens) | {M}):
        x = ctx.dev(inp["x"][:m])
        part = torch.empty(m, H, device="cuda")
        a_out = torch.empty(m, I_r, dtype=torch.bfloat16, device="cuda")

        def shard(i):
            rw = copies[(i // t) % copies_n][i % t]
            tp.tp_layer_shard_forward(desc, plans[i % t], tp.TP_STAGE_MLP, rw, x, part, ws=ws)

        def gateup(i):
            rw = copies[(i // t) % copies_n][i % t]
            tp.tp_column_linear(x, rw["w_gate"], a_out, w_up=rw["w_up"], gamma=gam, eps=wl.eps, ws=ws)

        for i in range(16):
            shard(i)
            gateup(i)
        s_mean, s_med, s_min = event_time_ms(torch, shard, nlaunch)
        k_mean, k_med, k_min = event_time_ms(torch, gateup, nlaunch)
        shard_bytes = 3 * I_r * H * 2 + m * H * 2 + H * 2 + m * H * 4
        gu_bytes = 2 * I_r * H * 2 + m * H * 2 + H * 2 + m * I_r * 2
        per_batch[m] = {
            "shard_us": s_mean * 1e3, "shard_us_median": s_med * 1e3, "shard_us_min": s_min * 1e3,
            "shard_bytes": shard_bytes, "shard_GBps": shard_bytes / (s_mean * 1e-3) / 1e9,
            "shard_pct_hbm_peak": 100 * shard_bytes / (s_mean * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "tokens_per_s_one_layer_shard": m / (s_mean * 1e-3),
            "gateup_kernel": projection_kernel(m, wide=True), "gateup_us": k_mean * 1e3, "gateup_us_median": k_med * 1e3,
            "gateup_us_min": k_min * 1e3, "gateup_bytes": gu_bytes, "gateup_GBps": gu_bytes / (k_mean * 1e-3) / 1e9,
            "_times": (k_mean, k_med, k_min),
        }
        log(f"[bench] m={m}: rank shard {s_mean * 1e3:.2f} us ({per_batch[m]['shard_GBps']:.0f} GB/s), "
            f"gate/up {k_mean * 1e3:.2f} us ({per_batch[m]['gateup_GBps']:.0f} GB/s)")

    x = ctx.dev(inp["x"][:M])
    parts = [torch.empty(M, H, device="cuda") for _ in range(t)]
    out = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")

    def step(i):
        ranks = copies[i % copies_n]
        for r, p in enumerate(plans):
            tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, ranks[r], x, parts[r], ws=ws)
        tp.tp_partial_sum(parts, out)

    total_ms = time_steps(ctx, step, copies_n)
    ms_step = total_ms / args.steps

    # The same step with bf16 row partials and their float32 sum (half the
    # bytes an all-reduce would move); the headline stays on float32 partials.
    a_bufs = [torch.empty(M, I_r, dtype=torch.bfloat16, device="cuda") for _ in range(t)]
    parts_b = [torch.empty(M, H, dtype=torch.bfloat16, device="cuda") for _ in range(t)]

    def step_bf16(i):
        ranks = copies[i % copies_n]
        for r in range(t):
            rw = ranks[r]
            tp.tp_column_linear(x, rw["w_gate"], a_bufs[r], w_up=rw["w_up"], gamma=gam, eps=wl.eps, ws=ws)
            tp.tp_row_linear_partial_bf16(a_bufs[r], rw["w_down"], parts_b[r], ws=ws)
        tp.tp_partial_sum_bf16(parts_b, out)

    total_b = time_steps(ctx, step_bf16, copies_n)
    hb = per_batch[M]
    k_mean, k_med, k_min = hb.pop("_times")
    for v in per_batch.values():
        v.pop("_times", None)
    extra = {
        "step_GBps": t * hb["shard_bytes"] / (ms_step * 1e-3) / 1e9,
        "per_rank_shard": {str(m): v for m, v in per_batch.items()},
        "bf16_partials": {"ms_per_step": total_b / args.steps, "tokens_per_s": M * args.steps / (total_b * 1e-3),
                          "partial_bytes_per_rank": M * H * 2},
        "roofline": roofline_hbm(projection_kernel(M, wide=True) + ": fused RMSNorm + gate/up + SwiGLU, one rank shard",
                                 f"gateup_mlp_decode_m{M}", hb["gateup_bytes"], k_mean, k_med, k_min),
    }
    config = {"workload": f"Llama-3-8B-shaped MLP decode block, all t={t} rank shards + on-device sum of partials",
              "hidden": H, "intermediate": I, "t": t, "tokens": M, "rmsnorm_eps": wl.eps,
              "weight_copies_rotated": copies_n}
    res = result(ctx, M * args.steps / (total_ms * 1e-3), "tokens/s", ms_step, config, extra)
    if not args.no_cpu:
        from oracle import sharded as S
        xs = inp["x"][:M]
        log(f"[bench] CPU oracle for ~{args.cpu_seconds:.0f} s")
        n, el = repeat_for(args.cpu_seconds, lambda: S.sharded_mlp(xs, inp["w_gate"], inp["w_up"], inp["w_down"], t,
                                                                    inp["gamma"], wl.eps))
        res["cpu_baseline"] = {"value": M * n / el, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
                               "sample": f"{n} full steps (all {t} rank shards in float64 + sum) of {M} tokens, "
                                         f"{el:.1f} s"}
    return res


def qkv_rank_phys(a, p, d):
    """The rank's fused QKV weight [q_cols + 2 kv_cols, H]: its q heads, then its k heads, then its v heads."""
    qb, qn, kb, kn = p.q_head_begin, p.q_heads, p.kv_head_begin, p.kv_heads
    return np.concatenate([a["w_q"][:, qb * d:(qb + qn) * d].T, a["w_k"][:, kb * d:(kb + kn) * d].T,
                           a["w_v"][:, kb * d:(kb + kn) * d].T], axis=0)


def bench_attn_proj(ctx):
    torch, tp, W, args = ctx.torch, ctx.tp, ctx.W, ctx.args
    wl = W.WORKLOADS[3]
    H, nq, nkv, d, t = wl.hidden, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t
    M = args.tokens or wl.tokens[0]
    copies_n = args.copies or 2
    log(f"[bench] drawing {wl.name}")
    a = W.attention_inputs(3, H, nq, nkv, d, M, 1, "bf16", with_cache=False)
    attn_in = W.attn_proj_input(3, M, nq * d, "bf16")
    desc = tp.make_desc(H, 0, nq, nkv, d)
    plans = [tp.tp_shard_plan(desc, t, r) for r in range(t)]
    x = ctx.dev(a["x"])
    copies = []
    for _ in range(copies_n):
        ranks = []
        for p in plans:
            qs = slice(p.q_head_begin * d, (p.q_head_begin + p.q_heads) * d)
            ranks.append({"w_qkv": ctx.dev(qkv_rank_phys(a, p, d)), "w_o": ctx.dev(ctx.phys(a["w_o"][qs, :])),
                          "attn": ctx.dev(attn_in[:, qs])})
        copies.append(ranks)
    qcols, orows = plans[0].qkv_cols, plans[0].o_rows
    ws = tp.workspace(max(tp.tp_linear_workspace_bytes(M, H, qcols, tp.TP_BF16, 0),
                          tp.tp_linear_workspace_bytes(M, orows, H, tp.TP_BF16, 0)))
    ys = [torch.empty(M, qcols, dtype=torch.bfloat16, device="cuda") for _ in range(t)]
    parts = [torch.empty(M, H, device="cuda") for _ in range(t)]
    out = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")

    def step(i):
        ranks = copies[i % copies_n]
        for r in range(t):
            tp.tp_column_linear(x, ranks[r]["w_qkv"], ys[r], ws=ws)
            tp.tp_row_linear_partial(ranks[r]["attn"], ranks[r]["w_o"], parts[r], ws=ws)
        tp.tp_partial_sum(parts, out)

    def qkv(i):
        rw = copies[(i // t) % copies_n][i % t]
        tp.tp_column_linear(x, rw["w_qkv"], ys[i % t], ws=ws)

    def wo(i):
        rw = copies[(i // t) % copies_n][i % t]
        tp.tp_row_linear_partial(rw["attn"], rw["w_o"], parts[i % t], ws=ws)

    for i in range(16):
        qkv(i)
        wo(i)
    nl = max(copies_n * t * 16, 64)
    q_t = event_time_ms(torch, qkv, nl)
    o_t = event_time_ms(torch, wo, nl)
    q_bytes = qcols * H * 2 + M * H * 2 + M * qcols * 2
    o_bytes = H * orows * 2 + M * orows * 2 + M * H * 4
    log(f"[bench] QKV {q_t[0] * 1e3:.2f} us ({q_bytes / (q_t[0] * 1e-3) / 1e9:.0f} GB/s), "
        f"W_o {o_t[0] * 1e3:.2f} us ({o_bytes / (o_t[0] * 1e-3) / 1e9:.0f} GB/s)")
    total_ms = time_steps(ctx, step, copies_n)
    ms_step = total_ms / args.steps
    rank_bytes = q_bytes + o_bytes
    extra = {
        "step_GBps": t * rank_bytes / (ms_step * 1e-3) / 1e9,
        "per_rank": {"qkv_us": q_t[0] * 1e3, "qkv_bytes": q_bytes, "qkv_GBps": q_bytes / (q_t[0] * 1e-3) / 1e9,
                     "wo_us": o_t[0] * 1e3, "wo_bytes": o_bytes, "wo_GBps": o_bytes / (o_t[0] * 1e-3) / 1e9,
                     "kernel": projection_kernel(M)},
        "roofline": roofline_hbm(projection_kernel(M) + ": QKV column projection, one rank shard",
                                 f"qkv_attn_proj_m{M}", q_bytes, *q_t),
    }
    config = {"workload": f"70B-shaped attention projections (QKV column + W_o row-partial), all t={t} rank shards "
                          f"+ on-device sum of partials", "hidden": H, "q_heads": nq, "kv_heads": nkv,
              "head_dim": d, "t": t, "tokens": M, "weight_copies_rotated": copies_n}
    res = result(ctx, M * args.steps / (total_ms * 1e-3), "tokens/s", ms_step, config, extra)
    if not args.no_cpu:
        from oracle import layer as L
        log(f"[bench] CPU oracle for ~{args.cpu_seconds:.0f} s")
        n, el = repeat_for(args.cpu_seconds, lambda: L.attn_proj_block(a["x"], attn_in, a["w_q"], a["w_k"], a["w_v"],
                                                                        a["w_o"]))
        res["cpu_baseline"] = {"value": M * n / el, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
                               "sample": f"{n} unsharded float64 projection blocks of {M} tokens (the sum of the "
                                         f"{t} shards' work), {el:.1f} s"}
    return res


def bench_mlp_prefill(ctx):
    torch, tp, W, args = ctx.torch, ctx.tp, ctx.W, ctx.args
    wl = W.WORKLOADS[4]
    H, I, t = wl.hidden, wl.intermediate, wl.t
    M = args.tokens or wl.tokens[0]
    log(f"[bench] drawing {wl.name}")
    inp = W.mlp_inputs(4, H, I, M, "bf16")
    desc = tp.make_desc(H, I)
    plans = [tp.tp_shard_plan(desc, t, r) for r in range(t)]
    I_r = plans[0].inter_cols
    ranks = []
    for p in plans:
        b, n = p.inter_begin, p.inter_cols
        ranks.append({"w_gate": ctx.dev(ctx.phys(inp["w_gate"][:, b:b + n])),
                      "w_up": ctx.dev(ctx.phys(inp["w_up"][:, b:b + n])),
                      "w_down": ctx.dev(ctx.phys(inp["w_down"][b:b + n]))})
    x = ctx.dev(inp["x"])
    ws = tp.workspace(max(tp.tp_layer_workspace_bytes(desc, p, tp.TP_STAGE_MLP, M, tp.TP_BF16) for p in plans))
    parts = [torch.empty(M, H, device="cuda") for _ in range(t)]
    out = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    a_out = torch.empty(M, I_r, dtype=torch.bfloat16, device="cuda")

    def step(i):
        for r, p in enumerate(plans):
            tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, ranks[r], x, parts[r], ws=ws)
        tp.tp_partial_sum(parts, out)

    def gateup(i):
        rw = ranks[i % t]
        tp.tp_column_linear(x, rw["w_gate"], a_out, w_up=rw["w_up"], ws=ws)

    def down(i):
        rw = ranks[i % t]
        tp.tp_row_linear_partial(a_out, rw["w_down"], parts[i % t], ws=ws)

    for i in range(4):
        gateup(i)
        down(i)
    g_t = event_time_ms(torch, gateup, 8, reps=3)
    d_t = event_time_ms(torch, down, 8, reps=3)
    g_fl, d_fl = 2.0 * M * H * 2 * I_r, 2.0 * M * I_r * H
    log(f"[bench] gate/up {g_t[0] * 1e3:.1f} us ({g_fl / (g_t[0] * 1e-3) / 1e12:.0f} TFLOP/s), "
        f"down {d_t[0] * 1e3:.1f} us ({d_fl / (d_t[0] * 1e-3) / 1e12:.0f} TFLOP/s)")
    total_ms = time_steps(ctx, step, 1)
    ms_step = total_ms / args.steps
    step_flops = t * (g_fl + d_fl)
    tflops = step_flops * args.steps / (total_ms * 1e-3) / 1e12
    g_tf = g_fl / (g_t[0] * 1e-3) / 1e12
    extra = {
        "tokens_per_s": M * args.steps / (total_ms * 1e-3),
        "pct_mfma_peak": 100 * tflops / BF16_PEAK_TFLOPS,
        "per_rank": {"gateup_us": g_t[0] * 1e3, "gateup_TFLOPs": g_tf, "down_us": d_t[0] * 1e3,
                     "down_TFLOPs": d_fl / (d_t[0] * 1e-3) / 1e12, "flops": g_fl + d_fl},
        "roofline": {"kernel": projection_kernel(M) + ": gate/up + SwiGLU, one rank shard", "bound": "mfma",
                     "achieved": g_tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": g_tf / BF16_PEAK_TFLOPS,
                     "traffic": counted_traffic(f"gateup_mlp_prefill_m{M}"), "flops_per_launch": g_fl,
                     "us_mean": g_t[0] * 1e3, "us_median": g_t[1] * 1e3, "us_min": g_t[2] * 1e3},
    }
    config = {"workload": f"70B-shaped MLP prefill block, all t={t} rank shards + on-device sum of partials",
              "hidden": H, "intermediate": I, "t": t, "tokens": M}
    res = result(ctx, tflops, "TFLOP/s", ms_step, config, extra)
    if not args.no_cpu:
        from oracle import sharded as S
        rows = 16
        xs = inp["x"][:rows]
        log(f"[bench] CPU oracle for ~{args.cpu_seconds:.0f} s")
        n, el = repeat_for(args.cpu_seconds, lambda: S.sharded_mlp(xs, inp["w_gate"], inp["w_up"], inp["w_down"], t))
        res["cpu_baseline"] = {"value": n * t * 2.0 * rows * 3 * H * I_r / el / 1e12, "unit": "TFLOP/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"{n} float64 steps (all {t} rank shards + sum) over the first {rows} of "
                                         f"the {M} tokens, {el:.1f} s"}
    return res


def bench_layer_decode(ctx):
    torch, tp, W, args = ctx.torch, ctx.tp, ctx.W, ctx.args
    wl = W.WORKLOADS[5]
    H, I, nq, nkv, d, t, S_ = wl.hidden, wl.intermediate, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t, wl.kv_len
    B = args.tokens or wl.tokens[0]
    log(f"[bench] drawing {wl.name}")
    a = W.attention_inputs(5, H, nq, nkv, d, B, S_, "bf16", "random")
    mi = W.mlp_inputs(5, H, I, B, "bf16", "random")
    desc = tp.make_desc(H, I, nq, nkv, d, n_layers=1, seq_len=S_, batch=B, eps=wl.eps)
    plans = [tp.tp_shard_plan(desc, t, r) for r in range(t)]
    g1, g2 = ctx.dev(a["gamma"]), ctx.dev(mi["gamma"])
    ranks = []
    for p in plans:
        qs = slice(p.q_head_begin * d, (p.q_head_begin + p.q_heads) * d)
        b, n = p.inter_begin, p.inter_cols
        kb, kn = p.kv_head_begin, p.kv_heads
        ranks.append({"attn_norm": g1, "w_qkv": ctx.dev(qkv_rank_phys(a, p, d)),
                      "w_o": ctx.dev(ctx.phys(a["w_o"][qs, :])), "mlp_norm": g2,
                      "w_gate": ctx.dev(ctx.phys(mi["w_gate"][:, b:b + n])),
                      "w_up": ctx.dev(ctx.phys(mi["w_up"][:, b:b + n])),
                      "w_down": ctx.dev(ctx.phys(mi["w_down"][b:b + n])),
                      "k": ctx.dev(a["k_cache"][:, kb:kb + kn]), "v": ctx.dev(a["v_cache"][:, kb:kb + kn])})
    x = ctx.dev(a["x"])
    ws = tp.workspace(max(max(tp.tp_layer_workspace_bytes(desc, p, tp.TP_STAGE_ATTN, B, tp.TP_BF16),
                              tp.tp_layer_workspace_bytes(desc, p, tp.TP_STAGE_MLP, B, tp.TP_BF16)) for p in plans))
    parts = [torch.empty(B, H, device="cuda") for _ in range(t)]
    h = torch.empty(B, H, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(B, H, dtype=torch.bfloat16, device="cuda")
    p0 = plans[0]
    q = torch.empty(B, p0.q_heads * d, dtype=torch.bfloat16, device="cuda").normal_()
    o = torch.empty_like(q)
    aw = tp.workspace(tp.tp_attention_workspace_bytes(B, p0.q_heads, p0.kv_heads, d, S_))

    def step(i):
        for r, p in enumerate(plans):
            rw = ranks[r]
            tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_ATTN, rw, x, parts[r],
                                      kv={"k": rw["k"], "v": rw["v"], "kv_len": S_}, ws=ws)
        tp.tp_partial_sum(parts, h, residual=x)
        for r, p in enumerate(plans):
            tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, ranks[r], h, parts[r], ws=ws)
        tp.tp_partial_sum(parts, out, residual=h)

    def attn(i):
        rw = ranks[i % t]
        tp.tp_decode_attention(q, rw["k"], rw["v"], o, S_, p0.q_heads, ws=aw)

    for i in range(16):
        attn(i)
    at = event_time_ms(torch, attn, max(4 * t, 32))
    kv_bytes = 2 * B * p0.kv_heads * S_ * d * 2 + 2 * B * p0.q_heads * d * 2
    log(f"[bench] attention {at[0] * 1e3:.2f} us ({kv_bytes / (at[0] * 1e-3) / 1e9:.0f} GB/s)")
    total_ms = time_steps(ctx, step, 1)
    ms_step = total_ms / args.steps
    w_rank = (p0.qkv_cols * H + H * p0.o_rows + 3 * p0.inter_cols * H) * 2
    kv_rank = 2 * B * p0.kv_heads * S_ * d * 2
    rank_bytes = w_rank + kv_rank
    extra = {
        "step_GBps": t * rank_bytes / (ms_step * 1e-3) / 1e9,
        "per_rank": {"weight_bytes": w_rank, "kv_bytes": kv_rank, "step_us_per_rank": ms_step * 1e3 / t,
                     "attention_us": at[0] * 1e3},
        "roofline": roofline_hbm("attn_decode_kernel + attn_merge_kernel (split-KV GQA decode attention, one rank)",
                                 f"attention_layer_decode_b{B}", kv_bytes, *at),
    }
    config = {"workload": f"70B-shaped full layer decode, all t={t} rank shards (attention and MLP stages) + "
                          f"on-device sums with residual", "hidden": H, "intermediate": I, "q_heads": nq,
              "kv_heads": nkv, "head_dim": d, "t": t, "batch": B, "kv_len": S_}
    # A model, not a measurement: the t-GPU decode step predicted from this
    # one-GPU layer time (all t shards run in turn) for 80 such layers.
    from megatron_tensor_transformer_amd import step_model
    extra["step_model_80_layers"] = step_model.predict(ms_step * 1e-3, layers=80, hidden=H, tokens=B, max_t=t)
    res = result(ctx, B * args.steps / (total_ms * 1e-3), "tokens/s", ms_step, config, extra)
    if not args.no_cpu:
        from oracle import sharded as S
        log(f"[bench] CPU oracle for ~{args.cpu_seconds:.0f} s")
        pd = tp.plan_dict(p0)
        xa = a["x"]

        def one_rank():
            S.rank_attention(xa, a["w_q"], a["w_k"], a["w_v"], a["w_o"], a["k_cache"], a["v_cache"], S_, nq, nkv, d,
                             pd, a["gamma"], wl.eps)
            S.rank_mlp(xa, mi["w_gate"], mi["w_up"], mi["w_down"], pd, mi["gamma"], wl.eps)

        n, el = repeat_for(args.cpu_seconds, one_rank)
        res["cpu_baseline"] = {"value": B * n / (el * t), "unit": "tokens/s", "cores": blas_threads(),
                               "kind": "oracle",
                               "sample": f"{n} float64 passes of rank 0's shard (attention + MLP stages) over the "
                                         f"batch of {B}, {el:.1f} s; scaled by 1/{t} for the {t} ranks of a step"}
    return res



def causal_flops(batch, seq, kv_len, q_heads, d):
    """Multiply-adds x 2 of causal attention: the token at position p scores and weights p + 1 keys."""
    p0 = kv_len - seq
    seen = seq * (p0 + 1) + seq * (seq - 1) // 2          # sum over the block of (p + 1)
    return 4.0 * d * batch * q_heads * seen


def bench_attn_prefill(ctx):
    torch, tp, W, args = ctx.torch, ctx.tp, ctx.W, ctx.args
    wl = W.WORKLOADS[6]
    nq, nkv, d, t, kv_len = wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t, wl.kv_len
    M = args.tokens or wl.tokens[0]
    B = 2
    S_ = M // B
    log(f"[bench] drawing {wl.name}")
    inp = W.prefill_attention_inputs(6, B, S_, nq, nkv, d, kv_len, "bf16")
    desc = tp.make_desc(wl.hidden, 0, nq, nkv, d, n_layers=1, seq_len=kv_len, batch=B)
    plans = [tp.tp_shard_plan(desc, t, r) for r in range(t)]
    q_all = inp["q"].reshape(B, S_, nq, d)
    ranks = []
    for p in plans:
        qb, qn, kb, kn = p.q_head_begin, p.q_heads, p.kv_head_begin, p.kv_heads
        ranks.append({"q": ctx.dev(q_all[:, :, qb:qb + qn].reshape(B, S_, qn * d)),
                      "k": ctx.dev(inp["k_cache"][:, kb:kb + kn]), "v": ctx.dev(inp["v_cache"][:, kb:kb + kn]),
                      "o": torch.empty(B, S_, qn * d, dtype=torch.bfloat16, device="cuda")})
    p0 = plans[0]

    def step(i):
        for r, p in enumerate(plans):
            rw = ranks[r]
            tp.tp_prefill_attention(rw["q"], rw["k"], rw["v"], rw["o"], kv_len, p.q_heads)

    def one(i):
        rw = ranks[i % t]
        tp.tp_prefill_attention(rw["q"], rw["k"], rw["v"], rw["o"], kv_len, p0.q_heads)

    for i in range(2 * t):
        one(i)
    at = event_time_ms(torch, one, 4 * t)
    fl = causal_flops(B, S_, kv_len, p0.q_heads, d)
    tf = fl / (at[0] * 1e-3) / 1e12
    log(f"[bench] prefill attention {at[0] * 1e3:.1f} us ({tf:.0f} TFLOP/s)")
    total_ms = time_steps(ctx, step, 1)
    ms_step = total_ms / args.steps
    tflops = t * fl * args.steps / (total_ms * 1e-3) / 1e12
    extra = {
        "tokens_per_s": M * args.steps / (total_ms * 1e-3),
        "pct_mfma_peak": 100 * tflops / BF16_PEAK_TFLOPS,
        "per_rank": {"attention_us": at[0] * 1e3, "causal_flops": fl},
        "roofline": {"kernel": "attn_prefill_kernel (causal GQA prefill attention, one rank shard)",
                     "bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / BF16_PEAK_TFLOPS, "traffic": counted_traffic(f"prefill_attention_m{M}"),
                     "flops_per_launch": fl, "us_mean": at[0] * 1e3, "us_median": at[1] * 1e3,
                     "us_min": at[2] * 1e3},
    }
    config = {"workload": f"70B-shaped causal prefill attention, all t={t} rank shards (each {p0.q_heads} q heads "
                          f"on {p0.kv_heads} kv head)", "q_heads": nq, "kv_heads": nkv, "head_dim": d, "t": t,
              "batch": B, "seq": S_, "kv_len": kv_len}
    res = result(ctx, tflops, "TFLOP/s", ms_step, config, extra)
    if not args.no_cpu:
        from oracle import sharded as S
        pd = tp.plan_dict(p0)
        n_tail = 32
        qs = inp["q"][:1, S_ - n_tail:].reshape(1, n_tail, nq, d)[:, :, p0.q_head_begin:p0.q_head_begin + p0.q_heads]
        qs = qs.reshape(1, n_tail, p0.q_heads * d)
        kr = inp["k_cache"][:1, p0.kv_head_begin:p0.kv_head_begin + p0.kv_heads]
        vr = inp["v_cache"][:1, p0.kv_head_begin:p0.kv_head_begin + p0.kv_heads]
        log(f"[bench] CPU oracle for ~{args.cpu_seconds:.0f} s")
        n, el = repeat_for(args.cpu_seconds, lambda: S.rank_prefill_attention(qs, kr, vr, kv_len, nq, nkv, d, pd))
        sfl = causal_flops(1, n_tail, kv_len, p0.q_heads, d)
        res["cpu_baseline"] = {"value": n * sfl / el / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
                               "kind": "oracle",
                               "sample": f"{n} float64 passes of rank 0's shard over the last {n_tail} tokens of "
                                         f"sequence 0 (each sees about {kv_len} keys), {el:.1f} s"}
    return res



def bench_layer_prefill(ctx):
    torch, tp, W, args = ctx.torch, ctx.tp, ctx.W, ctx.args
    wl = W.WORKLOADS[7]
    H, I, nq, nkv, d, t, kv_len = wl.hidden, wl.intermediate, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t, \
        wl.kv_len
    M = args.tokens or wl.tokens[0]
    B = 2
    S_ = M // B
    log(f"[bench] drawing {wl.name}")
    a = W.attention_inputs(7, H, nq, nkv, d, B, kv_len, "bf16", "random", with_cache=True)
    mi = W.mlp_inputs(7, H, I, 1, "bf16", "random")
    x_host = W.to_bf16(W.normal(7, W.Q_PREFILL, (B, S_, H)))
    desc = tp.make_desc(H, I, nq, nkv, d, n_layers=1, seq_len=kv_len, batch=B, eps=wl.eps)
    plans = [tp.tp_shard_plan(desc, t, r) for r in range(t)]
    g1, g2 = ctx.dev(a["gamma"]), ctx.dev(mi["gamma"])
    ranks = []
    for p in plans:
        qs = slice(p.q_head_begin * d, (p.q_head_begin + p.q_heads) * d)
        b0, n = p.inter_begin, p.inter_cols
        kb, kn = p.kv_head_begin, p.kv_heads
        ranks.append({"attn_norm": g1, "w_qkv": ctx.dev(qkv_rank_phys(a, p, d)),
                      "w_o": ctx.dev(ctx.phys(a["w_o"][qs, :])), "mlp_norm": g2,
                      "w_gate": ctx.dev(ctx.phys(mi["w_gate"][:, b0:b0 + n])),
                      "w_up": ctx.dev(ctx.phys(mi["w_up"][:, b0:b0 + n])),
                      "w_down": ctx.dev(ctx.phys(mi["w_down"][b0:b0 + n])),
                      "k": ctx.dev(a["k_cache"][:, kb:kb + kn]), "v": ctx.dev(a["v_cache"][:, kb:kb + kn])})
    x = ctx.dev(x_host.reshape(M, H))
    ws = tp.workspace(max(max(tp.tp_layer_workspace_bytes(desc, p, tp.TP_STAGE_ATTN, M, tp.TP_BF16),
                              tp.tp_layer_workspace_bytes(desc, p, tp.TP_STAGE_MLP, M, tp.TP_BF16)) for p in plans))
    parts = [torch.empty(M, H, device="cuda") for _ in range(t)]
    h = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    p0 = plans[0]
    a_out = torch.empty(M, p0.inter_cols, dtype=torch.bfloat16, device="cuda")
    hn = torch.empty(M, H, dtype=torch.bfloat16, device="cuda").normal_()

    def step(i):
        for r, p in enumerate(plans):
            rw = ranks[r]
            tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_ATTN, rw, x, parts[r],
                                      kv={"k": rw["k"], "v": rw["v"], "kv_len": kv_len, "new_tokens": S_}, ws=ws)
        tp.tp_partial_sum(parts, h, residual=x)
        for r, p in enumerate(plans):
            tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, ranks[r], h, parts[r], ws=ws)
        tp.tp_partial_sum(parts, out, residual=h)

    def gateup(i):
        rw = ranks[i % t]
        tp.tp_column_linear(hn, rw["w_gate"], a_out, w_up=rw["w_up"], ws=ws)

    for i in range(2 * t):
        gateup(i)
    g_t = event_time_ms(torch, gateup, 2 * t, reps=3)
    g_fl = 2.0 * M * H * 2 * p0.inter_cols
    g_tf = g_fl / (g_t[0] * 1e-3) / 1e12
    log(f"[bench] gate/up GEMM {g_t[0] * 1e3:.1f} us ({g_tf:.0f} TFLOP/s)")
    total_ms = time_steps(ctx, step, 1)
    ms_step = total_ms / args.steps
    rank_fl = (2.0 * M * H * p0.qkv_cols + causal_flops(B, S_, kv_len, p0.q_heads, d) + 2.0 * M * p0.o_rows * H
               + 2.0 * M * H * 3 * p0.inter_cols)
    tflops = t * rank_fl * args.steps / (total_ms * 1e-3) / 1e12
    extra = {
        "tokens_per_s": M * args.steps / (total_ms * 1e-3),
        "pct_mfma_peak": 100 * tflops / BF16_PEAK_TFLOPS,
        "per_rank": {"flops": rank_fl, "step_us_per_rank": ms_step * 1e3 / t, "gateup_us": g_t[0] * 1e3},
        "roofline": {"kernel": projection_kernel(M) + ": MLP gate/up + SwiGLU, one rank shard", "bound": "mfma",
                     "achieved": g_tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": g_tf / BF16_PEAK_TFLOPS,
                     "traffic": counted_traffic(f"gateup_layer_prefill_m{M}"), "flops_per_launch": g_fl,
                     "us_mean": g_t[0] * 1e3, "us_median": g_t[1] * 1e3, "us_min": g_t[2] * 1e3},
    }
    config = {"workload": f"70B-shaped full layer prefill, all t={t} rank shards (attention and MLP stages) + "
                          f"on-device sums with residual", "hidden": H, "intermediate": I, "q_heads": nq,
              "kv_heads": nkv, "head_dim": d, "t": t, "batch": B, "new_tokens": S_, "kv_len": kv_len}
    res = result(ctx, tflops, "TFLOP/s", ms_step, config, extra)
    if not args.no_cpu:
        from oracle import sharded as S
        pd = tp.plan_dict(p0)
        n_tail = 16
        xs = x_host[:1, S_ - n_tail:]
        log(f"[bench] CPU oracle for ~{args.cpu_seconds:.0f} s")

        def one_rank():
            at = S.rank_attention_prefill(xs, a["w_q"], a["w_k"], a["w_v"], a["w_o"], a["k_cache"][:1],
                                          a["v_cache"][:1], kv_len, nq, nkv, d, pd, a["gamma"], wl.eps)
            S.rank_mlp(xs.reshape(n_tail, H) + at["partial"].reshape(n_tail, H), mi["w_gate"], mi["w_up"],
                       mi["w_down"], pd, mi["gamma"], wl.eps)

        n, el = repeat_for(args.cpu_seconds, one_rank)
        sfl = (2.0 * n_tail * H * p0.qkv_cols + causal_flops(1, n_tail, kv_len, p0.q_heads, d)
               + 2.0 * n_tail * p0.o_rows * H + 2.0 * n_tail * H * 3 * p0.inter_cols)
        res["cpu_baseline"] = {"value": n * sfl / el / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
                               "kind": "oracle",
                               "sample": f"{n} float64 passes of rank 0's shard (attention and MLP stages) over "
                                         f"the last {n_tail} tokens of sequence 0 (each sees about {kv_len} keys), "
                                         f"{el:.1f} s"}
    return res



def bench_moe_decode(ctx):
    torch, tp, W, args = ctx.torch, ctx.tp, ctx.W, ctx.args
    wl = W.WORKLOADS[8]
    H, I, t, E, k = wl.hidden, wl.intermediate, wl.t, W.MOE_EXPERTS, W.MOE_TOP_K
    M = args.tokens or wl.tokens[0]
    log(f"[bench] drawing {wl.name}")
    inp = W.moe_inputs(8, H, I, E, M, "bf16", progress=lambda e: log(f"[bench]   expert {e} drawn"))
    desc = tp.make_desc(H, I)
    plans = [tp.tp_shard_plan(desc, t, r) for r in range(t)]
    cols = plans[0].inter_cols
    gam, rtr = ctx.dev(inp["gamma"]), ctx.dev(ctx.phys(inp["w_router"]))
    ranks = []
    for p in plans:
        b, c = p.inter_begin, p.inter_cols
        log(f"[bench] staging rank {p.rank}'s stacked experts")
        ranks.append({"norm": gam, "w_router": rtr,
                      "w_gate": ctx.dev(np.concatenate([ctx.phys(g[:, b:b + c]) for g, _, _ in inp["experts"]])),
                      "w_up": ctx.dev(np.concatenate([ctx.phys(u[:, b:b + c]) for _, u, _ in inp["experts"]])),
                      "w_down": ctx.dev(np.concatenate([ctx.phys(d[b:b + c]) for _, _, d in inp["experts"]],
                                                       axis=1))})
    x = ctx.dev(inp["x"])
    ws = tp.workspace(max(tp.tp_moe_workspace_bytes(M, H, E, cols, True),
                          tp.tp_linear_workspace_bytes(M, H, E * cols, tp.TP_BF16, tp.TP_LINEAR_SWIGLU)))
    parts = [torch.empty(M, H, device="cuda") for _ in range(t)]
    out = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    a_out = torch.empty(M, E * cols, dtype=torch.bfloat16, device="cuda")

    def step(i):
        for r in range(t):
            tp.tp_moe_shard_forward(ranks[r], x, parts[r], E, k, cols, eps=wl.eps, ws=ws)
        tp.tp_partial_sum(parts, out)

    def gateup(i):
        rw = ranks[i % t]
        tp.tp_column_linear(x, rw["w_gate"], a_out, w_up=rw["w_up"], ws=ws)

    for i in range(4 * t):
        gateup(i)
    g_t = event_time_ms(torch, gateup, 8 * t)
    g_bytes = 2 * E * cols * H * 2 + M * H * 2 + M * E * cols * 2
    log(f"[bench] stacked expert gate/up {g_t[0] * 1e3:.1f} us ({g_bytes / (g_t[0] * 1e-3) / 1e9:.0f} GB/s)")
    total_ms = time_steps(ctx, step, 1)
    ms_step = total_ms / args.steps
    rank_bytes = 3 * E * cols * H * 2 + E * H * 2
    extra = {
        "step_GBps": t * rank_bytes / (ms_step * 1e-3) / 1e9,
        "per_rank": {"weight_bytes": rank_bytes, "gateup_us": g_t[0] * 1e3, "experts": E, "top_k": k},
        "roofline": roofline_hbm(projection_kernel(M) + ": every expert's gate/up + SwiGLU (stacked), one rank shard",
                                 f"gateup_moe_decode_m{M}", g_bytes, *g_t),
    }
    config = {"workload": f"Mixtral-8x7B-shaped MoE FFN decode block, all t={t} rank shards + on-device sum",
              "hidden": H, "intermediate": I, "experts": E, "top_k": k, "t": t, "tokens": M}
    res = result(ctx, M * args.steps / (total_ms * 1e-3), "tokens/s", ms_step, config, extra)
    if not args.no_cpu:
        from oracle import layer as L
        from oracle import sharded as S
        n_tok = 4
        xs = inp["x"][:n_tok]
        log(f"[bench] CPU oracle for ~{args.cpu_seconds:.0f} s")

        def one_rank():
            gates = L.moe_route(L.linear(L.rmsnorm(xs, inp["gamma"], wl.eps), inp["w_router"]), k)
            S.rank_moe(xs, inp["gamma"], inp["w_router"], inp["experts"], gates, tp.plan_dict(plans[0]), wl.eps)

        n, el = repeat_for(args.cpu_seconds, one_rank)
        res["cpu_baseline"] = {"value": n_tok * n / (el * t), "unit": "tokens/s", "cores": blas_threads(),
                               "kind": "oracle",
                               "sample": f"{n} float64 passes of rank 0's MoE shard (router + all {E} experts) over "
                                         f"{n_tok} of the {M} tokens, {el:.1f} s; scaled by 1/{t} for the {t} ranks"}
    return res


if __name__ == "__main__":
    main()
