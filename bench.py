"""Throughput of one GPU's tensor-parallel layer shards on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mlp_decode|attn_proj|mlp_prefill|layer_decode]
                    [--tokens M] [--no-cpu]

Default workload: the Llama-3-8B-shaped MLP decode block (hidden 4096,
intermediate 14336, t=4, 16 tokens, RMSNorm in front). One step runs the
whole hot path on synthetic inputs already in HBM: every rank's shard (fused
RMSNorm + gate/up + SwiGLU, then the down row-partial) and the on-device sum
of the t partials. The weights are held in two copies that steps alternate
between, so the working set (704 MB) exceeds the 256 MB Infinity Cache and
weights stream from HBM.

Prints one JSON line. ``value`` is tokens per second of the whole step;
``roofline`` rates the dominant kernel (the fused gate/up projection) by its
algorithmic bytes over its average duration from per-launch HIP events on the
stream it runs on; ``cpu_baseline`` times the float64 CPU oracle on a bounded
sample of the same step.
"""
from __future__ import annotations

import argparse
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mlp_decode",
                    choices=["mlp_decode", "attn_proj", "mlp_prefill", "layer_decode"])
    ap.add_argument("--tokens", type=int, default=16, help="headline batch (the workload also times 1 and 4)")
    ap.add_argument("--copies", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's shard: only --gpus 1 is supported (the t rank shards of a layer run "
              "one after another on the single device and their partials are summed there).", file=sys.stderr)
        sys.exit(2)

    import torch

    import megatron_tensor_transformer_amd as tp
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    dev_name = torch.cuda.get_device_name(0)

    def dev(a, dt="bf16"):
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        return (t.to(torch.bfloat16) if dt == "bf16" else t).cuda()

    bench = {"mlp_decode": bench_mlp_decode}.get(args.workload)
    if bench is None:
        print(f"workload {args.workload} is not wired into bench.py yet", file=sys.stderr)
        sys.exit(2)
    res = bench(args, torch, tp, W, dev)
    res["device"] = dev_name
    print(json.dumps(res), flush=True)


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


def timed_replays(torch, graphs, steps):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gpu_hold(torch)
    e0.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def event_time_ms(torch, fn, n, reps=5):
    """Average ms per call of fn: n calls launched back to back between two HIP
    events on the stream they run on, repeated ``reps`` times.

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


def bench_mlp_decode(args, torch, tp, W, dev):
    wl = W.WORKLOADS[2]
    H, I, t, M = wl.hidden, wl.intermediate, wl.t, args.tokens
    log(f"[bench] drawing {wl.name}")
    inp = W.mlp_inputs(2, H, I, max(wl.tokens), "bf16", "ones")
    desc = tp.make_desc(H, I, eps=wl.eps)
    plans = [tp.tp_shard_plan(desc, t, r) for r in range(t)]
    I_r = plans[0].inter_cols
    gam = dev(inp["gamma"])
    copies = []
    for c in range(args.copies):
        ranks = []
        for p in plans:
            b, n = p.inter_begin, p.inter_cols
            ranks.append({"mlp_norm": gam,
                          "w_gate": dev(inp["w_gate"][:, b:b + n].T), "w_up": dev(inp["w_up"][:, b:b + n].T),
                          "w_down": dev(inp["w_down"][b:b + n].T)})
        copies.append(ranks)
    ws = tp.workspace(max(tp.tp_layer_workspace_bytes(desc, p, tp.TP_STAGE_MLP, max(wl.tokens), tp.TP_BF16)
                          for p in plans))
    nlaunch = max(len(copies) * t * 16, 64)

    def step_fn(x, parts, out):
        def step(i):
            ranks = copies[i % len(copies)]
            for r, p in enumerate(plans):
                tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, ranks[r], x, parts[r], ws=ws)
            tp.tp_partial_sum(parts, out)
        return step

    # one rank's shard and its dominant kernel, at every batch size of the workload
    per_batch = {}
    for m in sorted(set(wl.tokens) | {M}):
        x = dev(inp["x"][:m])
        part = torch.empty(m, H, device="cuda")
        a_out = torch.empty(m, I_r, dtype=torch.bfloat16, device="cuda")

        def shard(i):
            rw = copies[(i // t) % len(copies)][i % t]
            tp.tp_layer_shard_forward(desc, plans[i % t], tp.TP_STAGE_MLP, rw, x, part, ws=ws)

        def gateup(i):
            rw = copies[(i // t) % len(copies)][i % t]
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
            "gateup_us": k_mean * 1e3, "gateup_us_median": k_med * 1e3, "gateup_us_min": k_min * 1e3,
            "gateup_bytes": gu_bytes, "gateup_GBps": gu_bytes / (k_mean * 1e-3) / 1e9,
        }
        log(f"[bench] m={m}: rank shard {s_mean * 1e3:.2f} us ({per_batch[m]['shard_GBps']:.0f} GB/s), "
            f"gate/up {k_mean * 1e3:.2f} us ({per_batch[m]['gateup_GBps']:.0f} GB/s)")

    # the timed step at the headline batch: all t rank shards + the sum of partials
    x = dev(inp["x"][:M])
    parts = [torch.empty(M, H, device="cuda") for _ in range(t)]
    out = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    step = step_fn(x, parts, out)
    log(f"[bench] warmup {args.warmup} eager steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    graphs = capture_steps(torch, step, len(copies))
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} graph-replayed steps")
    total_ms = timed_replays(torch, graphs, args.steps)
    ms_step = total_ms / args.steps

    hb = per_batch[M]
    res = {
        "metric": METRIC,
        "value": M * args.steps / (total_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, gamma=1)",
        "config": {"workload": "Llama-3-8B-shaped MLP decode block, all t=4 rank shards + on-device sum of partials",
                   "hidden": H, "intermediate": I, "t": t, "tokens": M, "rmsnorm_eps": wl.eps,
                   "weight_copies_rotated": len(copies)},
        "step_GBps": 4 * hb["shard_bytes"] / (ms_step * 1e-3) / 1e9,
        "per_rank_shard": {str(m): v for m, v in per_batch.items()},
        "roofline": {"kernel": "gemv_kernel (fused RMSNorm + gate/up + SwiGLU column projection, one rank shard)",
                     "bound": "hbm", "achieved": hb["gateup_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": hb["gateup_GBps"] / HBM_PEAK_GBPS, "traffic": None,
                     "bytes_per_launch": hb["gateup_bytes"], "us_mean": hb["gateup_us"],
                     "us_median": hb["gateup_us_median"], "us_min": hb["gateup_us_min"]},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline_mlp({**inp, "x": inp["x"][:M]}, t, M, wl.eps, args.cpu_seconds)
    return res


def cpu_baseline_mlp(inp, t, M, eps, seconds):
    """The float64 oracle on the same step (all t rank shards + sum), repeated for about ``seconds``."""
    from oracle import sharded as S
    try:
        from threadpoolctl import threadpool_info
    except Exception:                      # pragma: no cover
        threadpool_info = None
    log(f"[bench] CPU oracle for ~{seconds:.0f} s")
    n = 0
    t0 = time.perf_counter()
    while True:
        S.sharded_mlp(inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"], t, inp["gamma"], eps)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    cores = None
    if threadpool_info is not None:
        th = [d.get("num_threads") for d in threadpool_info() if d.get("user_api") == "blas"]
        cores = max(th) if th else 1
    return {"value": M * n / el, "unit": "tokens/s", "cores": cores or 1, "kind": "oracle",
            "sample": f"{n} full steps (all {t} rank shards in float64 + sum) of {M} tokens, {el:.1f} s"}


if __name__ == "__main__":
    main()
