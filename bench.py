"""Throughput of one GPU's tensor-parallel layer shards on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--tokens M] [--no-cpu]

Workloads (synthetic, seeded inputs already in HBM; every rank shard of the
tensor-parallel group runs on the one device, then the on-device sum of the t
partials):

  headline (default)    the metric's two halves on their largest single-GPU
                        configurations, one JSON line: decode tokens/s and HBM
                        GB/s of the 70B-shaped full layer decode (below,
                        ``value``), and TFLOP/s of the 70B-shaped MLP prefill
                        (below, under ``prefill``), plus the streaming-read
                        rate of buffers the size of the decode launches.
  layer_decode          70B-shaped full layer, t=8, batch 16, KV cache of 8192
                        tokens: per rank RMSNorm + QKV (+ KV append), GQA decode
                        attention, W_o partial; sum + residual; RMSNorm +
                        gate/up + SwiGLU, down partial; sum + residual.
  mlp_prefill           70B-shaped MLP block, hidden 8192, intermediate 28672,
                        t=4, 4096 tokens (MFMA GEMMs); metric in TFLOP/s.
  mlp_decode            Llama-3-8B-shaped MLP block, hidden 4096, intermediate
                        14336, t=4, 16 tokens, RMSNorm in front: per rank fused
                        RMSNorm + gate/up + SwiGLU, then the down row-partial.
  attn_proj             70B-shaped attention projections, hidden 8192, 64 q / 8
                        kv heads of 128, t=4, 16 tokens: per rank the QKV column
                        projection and the W_o row-partial.
  attn_prefill, layer_prefill, moe_decode, moe_prefill
                        the prefill attention shard, the full layer over
                        2 x 2048 new tokens, the Mixtral-shaped MoE block at
                        16 decode tokens and at 4096 prefill tokens (each
                        expert over its routed tokens; TFLOP/s of routed flops).
  tiny_mlp              the tiny float32 MLP block (hidden 256, t=2, 4 tokens),
                        a correctness configuration; its time is launch-bound.
  hbm_read              the plain streaming-read rate alone.

One step is one pass of that whole path; K steps are replayed from HIP graphs
and timed between two events. Prints one JSON line. ``value`` is the step's
throughput; ``roofline`` rates the dominant kernel (the longest, measured) by
its algorithmic bytes (or flops) over its average duration, from HIP events
around back-to-back launches on the stream it runs on; ``cpu_baseline`` times
the float64 CPU oracle on a bounded sample of the same workload.

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
    ap.add_argument("--workload", default="headline",
                    choices=["headline", "mlp_decode", "attn_proj", "mlp_prefill", "layer_decode", "attn_prefill",
                             "layer_prefill", "moe_decode", "moe_prefill", "tiny_mlp", "hbm_read"])
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
    bench = {"headline": bench_headline, "hbm_read": bench_hbm_read, "mlp_decode": bench_mlp_decode, "attn_proj": bench_attn_proj, "mlp_prefill": bench_mlp_prefill,
             "layer_decode": bench_layer_decode, "attn_prefill": bench_attn_prefill,
             "layer_prefill": bench_layer_prefill, "moe_decode": bench_moe_decode,
             "moe_prefill": bench_moe_prefill, "tiny_mlp": bench_tiny_mlp}[args.workload]
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


class Marks:
    """HIP event pairs around the calls of a timed region's dominant kernels, by name, on torch's
    current stream (the stream the binding passes to every entry point)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def around(self, name, fn):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        self.pairs.setdefault(name, []).append((e0, e1))

    def stats(self, name):
        """(mean, median, min) ms per call over every marked call (after a synchronize)."""
        ms = [a.elapsed_time(b) for a, b in self.pairs[name]]
        return float(np.mean(ms)), float(np.median(ms)), float(np.min(ms)), len(ms)


def marked(mk, name, fn):
    if mk is None:
        fn()
    else:
        mk.around(name, fn)


def time_steps_eager(ctx, step):
    """Warm up eagerly, then time ``steps`` eager steps between two HIP events; ``step(i, marks)``
    records event pairs around its dominant calls, so their durations come from the timed region
    itself. For steps of milliseconds (the GEMM-bound prefill workloads), where launching from the host
    costs nothing against the kernels; steps of short kernels stay graph-replayed (time_steps). (Event
    nodes inside a captured graph, which would serve both, are refused by torch on ROCm.) Returns
    (total ms, Marks)."""
    torch, args = ctx.torch, ctx.args
    log(f"[bench] warmup {args.warmup} eager steps")
    for i in range(max(args.warmup, 1)):
        step(i, None)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} eager steps")
    marks = Marks(torch)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    gpu_hold(torch)
    e0.record()
    for i in range(args.steps):
        step(i, marks)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1), marks


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


def projection_kernel(m, dtype="bf16", wide=False, gemv_max_m=64):
    """The kernel a projection of m tokens runs on (the library's dispatch rule: the decode projections up
    to 64 tokens, or 16 for the stacked experts of an MoE decode batch); wide: one whose tiles fill the
    chip without splitting K (the 8B gate/up and down, the 70B W_o and t=8 MLP), which runs one K range
    per wave and, above 16 tokens, two blocks of 16 tokens per weight fetch."""
    if dtype == "bf16" and m > gemv_max_m:
        return "gemm_bf16_kernel (MFMA prefill GEMM)"
    if dtype == "bf16" and m >= 2:
        if wide and m > 16:
            return ("gemv_mfma_wide_kernel (matrix-core decode projection, one K range per wave, two 16-token "
                    "blocks per weight fetch)")
        if wide:
            return "gemv_mfma_wide_kernel (matrix-core decode projection, one K range per wave)"
        return "gemv_mfma_kernel (matrix-core decode projection)"
    return "gemv_kernel (v_dot2 decode projection)"


_KERNEL_DIGESTS = None


def kernel_digests():
    """Digest of each kernel's machine code in libtpshard.so, by kernel symbol: the gfx950 code objects
    in the .hip_fatbin section (clang offload bundles), each kernel's function bytes and its kernel
    descriptor (register, LDS and launch settings) without the descriptor's position-dependent code
    offset. A kernel keeps its digest while its own code is unchanged, whatever else is rebuilt."""
    global _KERNEL_DIGESTS
    if _KERNEL_DIGESTS is not None:
        return _KERNEL_DIGESTS
    import struct

    def sections(b):
        shoff = struct.unpack_from("<Q", b, 0x28)[0]
        shentsize, shnum, shstrndx = struct.unpack_from("<HHH", b, 0x3A)
        return [struct.unpack_from("<IIQQQQIIQQ", b, shoff + i * shentsize) for i in range(shnum)], shstrndx

    def cstr(b, at):
        return b[at:b.index(b"\0", at)]

    def code_object(co, out):
        secs, _ = sections(co)
        tabs = [x for x in secs if x[1] == 2]              # SHT_SYMTAB
        if not tabs:
            return
        st = tabs[0]
        strtab = secs[st[6]]
        funcs, descs = {}, {}
        for j in range(st[5] // 24):
            nm, info, _other, shndx, value, size = struct.unpack_from("<IBBHQQ", co, st[4] + j * 24)
            if shndx == 0 or shndx >= len(secs) or size == 0:
                continue
            name = cstr(co, strtab[4] + nm).decode()
            at = secs[shndx][4] + (value - secs[shndx][3])
            body = co[at:at + size]
            if info & 0xF == 2:                                 # STT_FUNC
                funcs[name] = body
            elif name.endswith(".kd") and size == 64:
                descs[name[:-3]] = body[:16] + b"\0" * 8 + body[24:]
        for name, body in funcs.items():
            out[name] = hashlib.sha256(body + descs.get(name, b"")).hexdigest()[:16]

    path = os.path.join(ROOT, "megatron_tensor_transformer_amd", "libtpshard.so")
    with open(path, "rb") as f:
        data = f.read()
    secs, shstrndx = sections(data)
    out = {}
    for name, _t, _f, _a, off, size, *_ in secs:
        if cstr(data, secs[shstrndx][4] + name) != b".hip_fatbin":
            continue
        fb = data[off:off + size]
        magic = b"__CLANG_OFFLOAD_BUNDLE__"
        i = fb.find(magic)
        while i >= 0:
            p = i + len(magic) + 8
            for _ in range(struct.unpack_from("<Q", fb, i + len(magic))[0]):
                eoff, esz, tsz = struct.unpack_from("<QQQ", fb, p)
                triple = fb[p + 24:p + 24 + tsz].decode()
                p += 24 + tsz
                if triple.endswith("gfx950") and esz:
                    code_object(fb[i + eoff:i + eoff + esz], out)
            i = fb.find(magic, i + 1)
    _KERNEL_DIGESTS = out
    return out


def code_digest(symbols):
    """One digest over the listed kernels' digests, or None if one is not in the library."""
    dig = kernel_digests()
    if not symbols or any(s not in dig for s in symbols):
        return None
    return hashlib.sha256(",".join(dig[s] for s in symbols).encode()).hexdigest()[:16]


def counted_traffic(kernel_key):
    """HBM bytes per launch of a kernel from the committed counter summary, or None.

    The summary holds, per (kernel, workload) key, FETCH_SIZE and WRITE_SIZE
    in KiB per dispatch from two counter runs, the kernels they cover (by
    symbol) with a digest of their machine code, and the same counters for the
    plain copy of known size that scales them to bytes. Figures taken on other
    code than the kernels loaded now are not used."""
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
    code = vals.get(f"{kernel_key}.code")
    if code is None or code != code_digest(vals.get(f"{kernel_key}.kernels", "").split()):
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


def time_legs(ctx, legs, unit, single_thread=()):
    """Time each CPU leg {name: (fn, units per run)} for a bounded share of --cpu-seconds on the BLAS
    threads, and the legs named in ``single_thread`` again on one thread."""
    from threadpoolctl import threadpool_limits
    runs = [(name, fn, per, None) for name, (fn, per) in legs.items()]
    runs += [(name + "_1thread", legs[name][0], legs[name][1], 1) for name in single_thread]
    share = ctx.args.cpu_seconds / len(runs)
    out = {}
    for name, fn, per, threads in runs:
        if threads is None:
            n, el = repeat_for(share, fn)
        else:
            with threadpool_limits(limits=threads):
                n, el = repeat_for(share, fn)
        out[name] = {unit: n * per / el, "runs": n, "seconds": el, "threads": threads or blas_threads()}
        log(f"[bench] CPU oracle {name}: {out[name][unit]:.4g} {unit}")
    return out


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
        from oracle import layer as L
        from oracle import plan as OP
        xs = inp["x"][:M]
        od = OP.ModelDesc(hidden=H, intermediate=I)

        def rank(r):
            op = OP.rank_plan(od, t, r)
            b, c = op["inter_begin"], op["inter_cols"]
            return L.mlp_block(xs, inp["w_gate"][:, b:b + c], inp["w_up"][:, b:b + c], inp["w_down"][b:b + c],
                               inp["gamma"], wl.eps)["y"]

        legs = time_legs(ctx, {"one_rank_shard": (lambda: rank(0), M),
                               "all_ranks_and_sum": (lambda: sum(rank(r) for r in range(t)), M),
                               "unsharded_block": (lambda: L.mlp_block(xs, inp["w_gate"], inp["w_up"], inp["w_down"],
                                                                       inp["gamma"], wl.eps)["y"], M)},
                         "tokens_per_s", single_thread=("one_rank_shard", "all_ranks_and_sum"))
        res["cpu_baseline"] = {"value": legs["all_ranks_and_sum"]["tokens_per_s"], "unit": "tokens/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"float64 oracle (BLAS products), the whole step: all {t} rank shards + sum "
                                         f"of {M} tokens; legs also one rank and the unsharded block, and on one "
                                         f"thread", "legs": legs, "host": host_info()}
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
        from oracle import plan as OP
        od = OP.ModelDesc(hidden=H, n_q_heads=nq, n_kv_heads=nkv, head_dim=d)

        def rank(r):
            op = OP.rank_plan(od, t, r)
            qs = slice(op["q_head_begin"] * d, (op["q_head_begin"] + op["q_heads"]) * d)
            ks = slice(op["kv_head_begin"] * d, (op["kv_head_begin"] + op["kv_heads"]) * d)
            return L.attn_proj_block(a["x"], attn_in[:, qs], a["w_q"][:, qs], a["w_k"][:, ks], a["w_v"][:, ks],
                                     a["w_o"][qs, :])["y"]

        legs = time_legs(ctx, {"one_rank_shard": (lambda: rank(0), M),
                               "all_ranks_and_sum": (lambda: sum(rank(r) for r in range(t)), M),
                               "unsharded_block": (lambda: L.attn_proj_block(a["x"], attn_in, a["w_q"], a["w_k"],
                                                                             a["w_v"], a["w_o"]), M)},
                         "tokens_per_s", single_thread=("one_rank_shard", "all_ranks_and_sum"))
        res["cpu_baseline"] = {"value": legs["all_ranks_and_sum"]["tokens_per_s"], "unit": "tokens/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"float64 oracle (BLAS products), the whole step: all {t} rank shards + sum "
                                         f"of {M} tokens; legs also one rank and the unsharded block, and on one "
                                         f"thread", "legs": legs, "host": host_info()}
    return res


def prefill_mlp_gpu(ctx):
    """The 70B-shaped MLP prefill block: all t rank shards + the sum, graph-replayed; the gate/up and
    down GEMMs of one rank timed with events. Returns (result fields, config, inputs)."""
    torch, tp, W, args = ctx.torch, ctx.tp, ctx.W, ctx.args
    wl = W.WORKLOADS[4]
    H, I, t = wl.hidden, wl.intermediate, wl.t
    M = args.tokens if (args.tokens and args.workload == "mlp_prefill") else wl.tokens[0]
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

    # A rank's MLP block: the gate/up + SwiGLU GEMM and the down GEMM (the MLP stage's two library
    # calls), each rank in turn, then the sum of the partials. The GEMMs are timed inside the timed
    # steps themselves.
    def step(i, mk=None):
        for r in range(t):
            rw = ranks[r]
            marked(mk, "gateup", lambda: tp.tp_column_linear(x, rw["w_gate"], a_out, w_up=rw["w_up"], ws=ws))
            marked(mk, "down", lambda: tp.tp_row_linear_partial(a_out, rw["w_down"], parts[r], ws=ws))
        tp.tp_partial_sum(parts, out)

    total_ms, mk = time_steps_eager(ctx, step)
    ms_step = total_ms / args.steps
    g_t, d_t = mk.stats("gateup"), mk.stats("down")
    g_fl, d_fl = 2.0 * M * H * 2 * I_r, 2.0 * M * I_r * H
    log(f"[bench] gate/up {g_t[0] * 1e3:.1f} us ({g_fl / (g_t[0] * 1e-3) / 1e12:.0f} TFLOP/s), "
        f"down {d_t[0] * 1e3:.1f} us ({d_fl / (d_t[0] * 1e-3) / 1e12:.0f} TFLOP/s), over {g_t[3]} calls each")
    step_flops = t * (g_fl + d_fl)
    tflops = step_flops * args.steps / (total_ms * 1e-3) / 1e12
    g_tf = g_fl / (g_t[0] * 1e-3) / 1e12
    fields = {
        "tflops": tflops, "ms_per_step": ms_step,
        "tokens_per_s": M * args.steps / (total_ms * 1e-3),
        "pct_mfma_peak": 100 * tflops / BF16_PEAK_TFLOPS,
        "step_flops": step_flops,
        "per_rank": {"gateup_us": g_t[0] * 1e3, "gateup_TFLOPs": g_tf, "down_us": d_t[0] * 1e3,
                     "down_TFLOPs": d_fl / (d_t[0] * 1e-3) / 1e12, "flops": g_fl + d_fl},
        "roofline": {"kernel": projection_kernel(M) + ": gate/up + SwiGLU, one rank shard (one library call: "
                               "the GEMM and the tail of its last round)", "bound": "mfma",
                     "achieved": g_tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": g_tf / BF16_PEAK_TFLOPS,
                     "traffic": counted_traffic(f"gateup_mlp_prefill_m{M}"), "flops_per_launch": g_fl,
                     "us_mean": g_t[0] * 1e3, "us_median": g_t[1] * 1e3, "us_min": g_t[2] * 1e3,
                     "timed": f"every gate/up call of the {args.steps} timed steps ({g_t[3]} calls)"},
    }
    config = {"workload": f"70B-shaped MLP prefill block, all t={t} rank shards + on-device sum of partials",
              "hidden": H, "intermediate": I, "t": t, "tokens": M}
    return fields, config, inp


def prefill_mlp_cpu(ctx, inp, rows=256):
    """The float64 oracle on the prefill MLP block over the first ``rows`` tokens: (i) one rank's shard,
    (ii) all t shards + the rank-order sum, (iii) the unsharded block; TFLOP/s of each."""
    from oracle import layer as L
    from oracle import plan as OP
    wl = ctx.W.WORKLOADS[4]
    H, I, t = wl.hidden, wl.intermediate, wl.t
    xs = inp["x"][:rows]
    od = OP.ModelDesc(hidden=H, intermediate=I)

    def rank(r):
        op = OP.rank_plan(od, t, r)
        b, c = op["inter_begin"], op["inter_cols"]
        return L.mlp_block(xs, inp["w_gate"][:, b:b + c], inp["w_up"][:, b:b + c], inp["w_down"][b:b + c])["y"]

    fl_all = 6.0 * rows * H * I
    legs = {
        "one_rank_shard": (lambda: rank(0), fl_all / t),
        "all_ranks_and_sum": (lambda: sum(rank(r) for r in range(t)), fl_all),
        "unsharded_block": (lambda: L.mlp_block(xs, inp["w_gate"], inp["w_up"], inp["w_down"])["y"], fl_all),
    }
    out = {}
    for name, (fn, fl) in legs.items():
        n, el = repeat_for(ctx.args.cpu_seconds / 3, fn)
        out[name] = {"TFLOPs": n * fl / el / 1e12, "runs": n, "seconds": el, "flops_per_run": fl}
        log(f"[bench] CPU oracle, prefill MLP {name}: {out[name]['TFLOPs'] * 1e3:.2f} GFLOP/s")
    return out, f"the first {rows} of the {inp['x'].shape[0]} tokens"


def bench_mlp_prefill(ctx):
    fields, config, inp = prefill_mlp_gpu(ctx)
    extra = {k: v for k, v in fields.items() if k not in ("tflops", "ms_per_step")}
    res = result(ctx, fields["tflops"], "TFLOP/s", fields["ms_per_step"], config, extra)
    if not ctx.args.no_cpu:
        legs, sample = prefill_mlp_cpu(ctx, inp)
        res["cpu_baseline"] = {"value": legs["all_ranks_and_sum"]["TFLOPs"], "unit": "TFLOP/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"float64 oracle, all {config['t']} rank shards + sum over {sample}",
                               "legs": legs, "host": host_info()}
    return res


def decode_layer_gpu(ctx):
    """The 70B-shaped layer decode (t=8, batch 16, KV 8192): every rank's attention stage, the sum with the
    residual, every rank's MLP stage, the sum with the residual, graph-replayed. One rank's shard and each
    of its projections and its attention are also timed with events, rotating over the t ranks' weights.
    Returns (result fields, config, inputs)."""
    torch, tp, W, args = ctx.torch, ctx.tp, ctx.W, ctx.args
    wl = W.WORKLOADS[5]
    H, I, nq, nkv, d, t, S_ = wl.hidden, wl.intermediate, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t, wl.kv_len
    B = args.tokens if (args.tokens and args.workload == "layer_decode") else wl.tokens[0]
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
    qc, orows, I_r, kv_r, q_r = p0.qkv_cols, p0.o_rows, p0.inter_cols, p0.kv_heads, p0.q_heads

    def step(i):
        for r, p in enumerate(plans):
            rw = ranks[r]
            tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_ATTN, rw, x, parts[r],
                                      kv={"k": rw["k"], "v": rw["v"], "kv_len": S_}, ws=ws)
        tp.tp_partial_sum(parts, h, residual=x)
        for r, p in enumerate(plans):
            tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, ranks[r], h, parts[r], ws=ws)
        tp.tp_partial_sum(parts, out, residual=h)

    # one rank's pieces, each rotating over the t ranks' weights (2.3 GB in all: HBM, not the cache)
    yq = torch.empty(B, qc, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(B, orows, dtype=torch.bfloat16, device="cuda").normal_()
    o = torch.empty_like(q)
    act = torch.empty(B, I_r, dtype=torch.bfloat16, device="cuda")
    part = torch.empty(B, H, device="cuda")
    hn = torch.empty(B, H, dtype=torch.bfloat16, device="cuda").normal_()
    aw = tp.workspace(tp.tp_attention_workspace_bytes(B, q_r, kv_r, d, S_))

    def shard(i):
        rw, p = ranks[i % t], plans[i % t]
        tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_ATTN, rw, x, parts[i % t],
                                  kv={"k": rw["k"], "v": rw["v"], "kv_len": S_}, ws=ws)
        tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, rw, hn, parts[i % t], ws=ws)

    pieces = {
        "qkv": (lambda i: tp.tp_column_linear(x, ranks[i % t]["w_qkv"], yq, gamma=g1, eps=wl.eps, ws=ws),
                qc * H * 2 + B * H * 2 + H * 2 + B * qc * 2,
                projection_kernel(B) + " + merge: RMSNorm + QKV column projection"),
        "attention": (lambda i: tp.tp_decode_attention(q, ranks[i % t]["k"], ranks[i % t]["v"], o, S_, q_r, ws=aw),
                      2 * B * kv_r * S_ * d * 2 + 2 * B * q_r * d * 2,
                      "attn_decode_kernel + attn_merge_kernel: split-KV GQA decode attention"),
        "w_o": (lambda i: tp.tp_row_linear_partial(o, ranks[i % t]["w_o"], part, ws=ws),
                H * orows * 2 + B * orows * 2 + B * H * 4,
                projection_kernel(B, wide=True) + ": W_o row partial"),
        "gate_up": (lambda i: tp.tp_column_linear(hn, ranks[i % t]["w_gate"], act, w_up=ranks[i % t]["w_up"], gamma=g2,
                                                  eps=wl.eps, ws=ws),
                    2 * I_r * H * 2 + B * H * 2 + H * 2 + B * I_r * 2,
                    projection_kernel(B, wide=True) + ": RMSNorm + gate/up + SwiGLU"),
        "down": (lambda i: tp.tp_row_linear_partial(act, ranks[i % t]["w_down"], part, ws=ws),
                 H * I_r * 2 + B * I_r * 2 + B * H * 4,
                 projection_kernel(B, wide=True) + ": down row partial"),
    }
    nl = 4 * t
    kernels = {}
    for name, (fn, nbytes, kname) in pieces.items():
        for i in range(2 * t):
            fn(i)
        tm = event_time_ms(torch, fn, nl)
        kernels[name] = roofline_hbm(kname + ", one rank", f"{name}_layer_decode_b{B}", nbytes, *tm)
        log(f"[bench] {name}: {tm[0] * 1e3:.2f} us ({kernels[name]['achieved']:.0f} GB/s)")
    for i in range(2 * t):
        shard(i)
    sh = event_time_ms(torch, shard, nl)
    w_rank = (qc * H + H * orows + 3 * I_r * H) * 2
    kv_rank = 2 * B * kv_r * S_ * d * 2
    io_rank = 2 * B * H * 2 + 2 * B * H * 4 + 2 * H * 2 + 2 * B * kv_r * d * 2
    rank_bytes = w_rank + kv_rank + io_rank
    log(f"[bench] rank shard: {sh[0] * 1e3:.2f} us ({rank_bytes / (sh[0] * 1e-3) / 1e9:.0f} GB/s)")
    total_ms = time_steps(ctx, step, 1)
    ms_step = total_ms / args.steps
    dom = max(kernels, key=lambda k: kernels[k]["us_mean"])
    from megatron_tensor_transformer_amd import step_model
    fields = {
        "tokens_per_s": B * args.steps / (total_ms * 1e-3), "ms_per_step": ms_step,
        "step_GBps": t * rank_bytes / (ms_step * 1e-3) / 1e9,
        "step_pct_hbm_peak": 100 * t * rank_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "rank_shard": {"bytes": rank_bytes, "weight_bytes": w_rank, "kv_bytes": kv_rank, "io_bytes": io_rank,
                       "us_mean": sh[0] * 1e3, "us_median": sh[1] * 1e3, "us_min": sh[2] * 1e3,
                       "GBps": rank_bytes / (sh[0] * 1e-3) / 1e9,
                       "pct_hbm_peak": 100 * rank_bytes / (sh[0] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                       "tokens_per_s_one_layer_shard": B / (sh[0] * 1e-3)},
        "kernels": kernels,
        "dominant_kernel": dom,
        "roofline": kernels[dom],
        # extrapolation, not a measurement: 80 such layers, all t shards on one GPU in turn
        "extrapolated_80_layer_tokens_per_s": B / (80 * ms_step * 1e-3),
        # a model, not a measurement: the t-GPU step predicted from this one-GPU layer time
        "step_model_80_layers": step_model.predict(ms_step * 1e-3, layers=80, hidden=H, tokens=B, max_t=t),
    }
    config = {"workload": f"70B-shaped full layer decode, all t={t} rank shards (attention and MLP stages) + "
                          f"on-device sums with residual", "hidden": H, "intermediate": I, "q_heads": nq,
              "kv_heads": nkv, "head_dim": d, "t": t, "batch": B, "kv_len": S_}
    return fields, config, (a, mi)


def decode_layer_cpu(ctx, inputs):
    """The float64 oracle on the 70B-shaped layer decode step (all 16 tokens): (i) one rank's shard (its
    attention and MLP blocks on its own heads and columns), (ii) all t shards with the rank-order sums
    and residuals, (iii) the unsharded layer; tokens/s of each."""
    from oracle import layer as L
    from oracle import plan as OP
    a, mi = inputs
    wl = ctx.W.WORKLOADS[5]
    H, I, nq, nkv, d, t, S_ = wl.hidden, wl.intermediate, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.t, wl.kv_len
    B = a["x"].shape[0]
    od = OP.ModelDesc(hidden=H, intermediate=I, n_q_heads=nq, n_kv_heads=nkv, head_dim=d, seq_len=S_, batch=B)
    ops = [OP.rank_plan(od, t, r) for r in range(t)]

    def attn_rank(op, x):
        qs = slice(op["q_head_begin"] * d, (op["q_head_begin"] + op["q_heads"]) * d)
        ks = slice(op["kv_head_begin"] * d, (op["kv_head_begin"] + op["kv_heads"]) * d)
        hs = slice(op["kv_head_begin"], op["kv_head_begin"] + op["kv_heads"])
        return L.attention_block(x, a["w_q"][:, qs], a["w_k"][:, ks], a["w_v"][:, ks], a["w_o"][qs, :],
                                 a["k_cache"][:, hs], a["v_cache"][:, hs], S_, op["q_heads"], op["kv_heads"], d,
                                 a["gamma"], wl.eps)["y"]

    def mlp_rank(op, h):
        b, c = op["inter_begin"], op["inter_cols"]
        return L.mlp_block(h, mi["w_gate"][:, b:b + c], mi["w_up"][:, b:b + c], mi["w_down"][b:b + c],
                           mi["gamma"], wl.eps)["y"]

    def one_rank():
        mlp_rank(ops[0], L.f64(a["x"]) + attn_rank(ops[0], a["x"]))

    def all_ranks():
        h = L.f64(a["x"]) + sum(attn_rank(op, a["x"]) for op in ops)
        return h + sum(mlp_rank(op, h) for op in ops)

    w = {"gamma1": a["gamma"], "w_q": a["w_q"], "w_k": a["w_k"], "w_v": a["w_v"], "w_o": a["w_o"],
         "gamma2": mi["gamma"], "w_gate": mi["w_gate"], "w_up": mi["w_up"], "w_down": mi["w_down"]}
    legs = {"one_rank_shard": one_rank, "all_ranks_and_sums": all_ranks,
            "unsharded_layer": lambda: L.layer(a["x"], w, a["k_cache"], a["v_cache"], S_, nq, nkv, d, wl.eps)}
    out = {}
    for name, fn in legs.items():
        n, el = repeat_for(ctx.args.cpu_seconds / 3, fn)
        out[name] = {"tokens_per_s": B * n / el, "runs": n, "seconds": el}
        log(f"[bench] CPU oracle, layer decode {name}: {out[name]['tokens_per_s']:.1f} tokens/s")
    return out


def host_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cpus_available": len(os.sched_getaffinity(0)), "blas_threads": blas_threads()}


def bench_layer_decode(ctx):
    fields, config, inputs = decode_layer_gpu(ctx)
    extra = {k: v for k, v in fields.items() if k not in ("tokens_per_s", "ms_per_step")}
    res = result(ctx, fields["tokens_per_s"], "tokens/s", fields["ms_per_step"], config, extra)
    if not ctx.args.no_cpu:
        legs = decode_layer_cpu(ctx, inputs)
        res["cpu_baseline"] = {"value": legs["all_ranks_and_sums"]["tokens_per_s"], "unit": "tokens/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": "float64 oracle (BLAS products), the whole step: all 8 rank shards + "
                                         "sums + residuals over the batch of 16", "legs": legs, "host": host_info()}
    return res


def hbm_read_ceiling(ctx, sizes=(58_974_208, 117_833_728, 1 << 30)):
    """The plain streaming-read rate of buffers the size of the decode launches (and 1 GiB), each
    buffer read once per launch, rotating over enough copies to stay out of the 256 MB cache."""
    torch, tp = ctx.torch, ctx.tp
    flag = torch.zeros(4, dtype=torch.int32, device="cuda")
    out = {}
    for nb in sizes:
        copies = max(2, -(-(768 << 20) // nb))
        bufs = [torch.empty(nb // 4, dtype=torch.int32, device="cuda").fill_(i + 1) for i in range(copies)]

        def rd(i):
            tp.tp_hbm_stream_read(bufs[i % copies], flag)

        for i in range(2 * copies):
            rd(i)
        n = max(4 * copies, 16) if nb < (1 << 28) else 8
        tm = event_time_ms(torch, rd, n)
        out[str(nb)] = {"GBps": nb / (tm[0] * 1e-3) / 1e9, "us_mean": tm[0] * 1e3, "us_min": tm[2] * 1e3,
                        "buffers_rotated": copies}
        log(f"[bench] streaming read of {nb / 1e6:.1f} MB: {out[str(nb)]['GBps']:.0f} GB/s")
        del bufs
    torch.cuda.synchronize()
    return out


def bench_hbm_read(ctx):
    """The streaming-read reference alone."""
    ceiling = hbm_read_ceiling(ctx)
    big = ceiling[str(1 << 30)]
    config = {"workload": "plain streaming read of device buffers (1 GiB and decode-launch sizes)"}
    return result(ctx, big["GBps"], "GB/s", big["us_mean"] * 1e-3, config, {"hbm_read_ceiling": ceiling})


def bench_headline(ctx):
    """The metric's two halves on their largest single-GPU configurations: the 70B-shaped full layer
    decode shard (t=8, batch 16, KV 8192) for decode tokens/s and HBM GB/s, and the 70B-shaped MLP
    prefill shard (t=4, 4096 tokens) for TFLOP/s against the bf16 matrix-core peak."""
    args = ctx.args
    dec, dcfg, dinputs = decode_layer_gpu(ctx)
    pre, pcfg, pinp = prefill_mlp_gpu(ctx)
    ceiling = hbm_read_ceiling(ctx)
    config = {"workload": "70B-shaped full layer decode shard (t=8, batch 16, KV cache 8192; all 8 rank shards "
                          "+ on-device sums) and 70B-shaped MLP prefill shard (t=4, 4096 tokens; all 4 rank shards "
                          "+ on-device sum)",
              "decode": dcfg, "prefill": pcfg}
    extra = {k: v for k, v in dec.items() if k not in ("tokens_per_s", "ms_per_step")}
    extra["prefill"] = pre
    extra["prefill_ms_per_step"] = pre["ms_per_step"]
    extra["hbm_read_ceiling"] = ceiling
    res = result(ctx, dec["tokens_per_s"], "tokens/s", dec["ms_per_step"], config, extra)
    if not args.no_cpu:
        dlegs = decode_layer_cpu(ctx, dinputs)
        plegs, psample = prefill_mlp_cpu(ctx, pinp)
        res["cpu_baseline"] = {"value": dlegs["all_ranks_and_sums"]["tokens_per_s"], "unit": "tokens/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": "float64 oracle with BLAS products on the decode step: all 8 rank shards "
                                         "+ sums + residuals over the batch of 16 (legs: one rank's shard, all "
                                         "ranks, the unsharded layer); prefill legs over " + psample,
                               "legs": dlegs, "prefill_legs": plegs, "host": host_info()}
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

    # A step is the t ranks' attention calls back to back, replayed from a graph (the calls are too
    # short for eager launches to keep up); every call of the timed region is the dominant kernel, so
    # its average duration is the timed region's time over its calls.
    def step(i):
        for r, p in enumerate(plans):
            rw = ranks[r]
            tp.tp_prefill_attention(rw["q"], rw["k"], rw["v"], rw["o"], kv_len, p.q_heads)

    def one(i):
        rw = ranks[i % t]
        tp.tp_prefill_attention(rw["q"], rw["k"], rw["v"], rw["o"], kv_len, p0.q_heads)

    total_ms = time_steps(ctx, step, 1)
    ms_step = total_ms / args.steps
    n_calls = args.steps * t
    bb = event_time_ms(torch, one, 4 * t)           # back to back, outside the timed region: for reference
    at = (total_ms / n_calls, total_ms / n_calls, total_ms / n_calls, n_calls)
    fl = causal_flops(B, S_, kv_len, p0.q_heads, d)
    tf = fl / (at[0] * 1e-3) / 1e12
    log(f"[bench] prefill attention {at[0] * 1e3:.1f} us ({tf:.0f} TFLOP/s) per call in the timed steps, "
        f"{bb[0] * 1e3:.1f} us back to back")
    tflops = t * fl * args.steps / (total_ms * 1e-3) / 1e12
    extra = {
        "tokens_per_s": M * args.steps / (total_ms * 1e-3),
        "pct_mfma_peak": 100 * tflops / BF16_PEAK_TFLOPS,
        "per_rank": {"attention_us": at[0] * 1e3, "causal_flops": fl},
        "roofline": {"kernel": "attn_prefill_kernel (causal GQA prefill attention, one rank shard)",
                     "bound": "mfma", "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / BF16_PEAK_TFLOPS, "traffic": counted_traffic(f"prefill_attention_m{M}"),
                     "flops_per_launch": fl, "us_mean": at[0] * 1e3,
                     "timed": f"the timed region's {args.steps} graph-replayed steps over their {n_calls} calls "
                              f"(every call is this kernel; gaps between calls included)",
                     "us_back_to_back": bb[0] * 1e3},
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
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):     # the sharded oracle's einsum products run on one thread
            n, el = repeat_for(args.cpu_seconds, lambda: S.rank_prefill_attention(qs, kr, vr, kv_len, nq, nkv, d,
                                                                                  pd))
        sfl = causal_flops(1, n_tail, kv_len, p0.q_heads, d)
        res["cpu_baseline"] = {"value": n * sfl / el / 1e12, "unit": "TFLOP/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{n} float64 passes (sharded oracle, numpy einsum on one thread) of rank 0's "
                                         f"shard over the last {n_tail} tokens of "
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

    # The attention stage of every rank, the sum, then every rank's MLP block as the MLP stage's two
    # library calls (RMSNorm + gate/up + SwiGLU, then down), so the gate/up call is timed inside the
    # timed steps; then the second sum.
    def step(i, mk=None):
        for r, p in enumerate(plans):
            rw = ranks[r]
            tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_ATTN, rw, x, parts[r],
                                      kv={"k": rw["k"], "v": rw["v"], "kv_len": kv_len, "new_tokens": S_}, ws=ws)
        tp.tp_partial_sum(parts, h, residual=x)
        for r in range(t):
            rw = ranks[r]
            marked(mk, "gateup", lambda: tp.tp_column_linear(h, rw["w_gate"], a_out, w_up=rw["w_up"],
                                                             gamma=rw["mlp_norm"], eps=wl.eps, ws=ws))
            tp.tp_row_linear_partial(a_out, rw["w_down"], parts[r], ws=ws)
        tp.tp_partial_sum(parts, out, residual=h)

    total_ms, mk = time_steps_eager(ctx, step)
    ms_step = total_ms / args.steps
    g_t = mk.stats("gateup")
    g_fl = 2.0 * M * H * 2 * p0.inter_cols
    g_tf = g_fl / (g_t[0] * 1e-3) / 1e12
    log(f"[bench] RMSNorm + gate/up GEMM {g_t[0] * 1e3:.1f} us ({g_tf:.0f} TFLOP/s) over {g_t[3]} calls")
    rank_fl = (2.0 * M * H * p0.qkv_cols + causal_flops(B, S_, kv_len, p0.q_heads, d) + 2.0 * M * p0.o_rows * H
               + 2.0 * M * H * 3 * p0.inter_cols)
    tflops = t * rank_fl * args.steps / (total_ms * 1e-3) / 1e12
    extra = {
        "tokens_per_s": M * args.steps / (total_ms * 1e-3),
        "pct_mfma_peak": 100 * tflops / BF16_PEAK_TFLOPS,
        "per_rank": {"flops": rank_fl, "step_us_per_rank": ms_step * 1e3 / t, "gateup_us": g_t[0] * 1e3},
        "roofline": {"kernel": projection_kernel(M) + ": MLP gate/up + SwiGLU, one rank shard (one library call: "
                               "rmsnorm_kernel, then the GEMM; the RMSNorm's flops are not counted)", "bound": "mfma",
                     "achieved": g_tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": g_tf / BF16_PEAK_TFLOPS,
                     "traffic": counted_traffic(f"gateup_layer_prefill_m{M}"), "flops_per_launch": g_fl,
                     "us_mean": g_t[0] * 1e3, "us_median": g_t[1] * 1e3, "us_min": g_t[2] * 1e3,
                     "timed": f"every MLP gate/up call of the {args.steps} timed steps ({g_t[3]} calls)"},
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

        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):     # the sharded oracle's einsum products run on one thread
            n, el = repeat_for(args.cpu_seconds, one_rank)
        sfl = (2.0 * n_tail * H * p0.qkv_cols + causal_flops(1, n_tail, kv_len, p0.q_heads, d)
               + 2.0 * n_tail * p0.o_rows * H + 2.0 * n_tail * H * 3 * p0.inter_cols)
        res["cpu_baseline"] = {"value": n * sfl / el / 1e12, "unit": "TFLOP/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{n} float64 passes (sharded oracle, numpy einsum on one thread) of rank "
                                         f"0's shard (attention and MLP stages) over "
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
    ws = tp.workspace(max(tp.tp_moe_workspace_bytes(M, H, E, k, cols, True),
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
        "roofline": roofline_hbm(projection_kernel(M, gemv_max_m=16) + ": every expert's gate/up + SwiGLU (stacked), "
                                 "one rank shard",
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

        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):     # the sharded oracle's einsum products run on one thread
            n, el = repeat_for(args.cpu_seconds, one_rank)
        res["cpu_baseline"] = {"value": n_tok * n / (el * t), "unit": "tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{n} float64 passes (sharded oracle, numpy einsum on one thread) of rank 0's MoE shard (router + all {E} experts) over "
                                         f"{n_tok} of the {M} tokens, {el:.1f} s; scaled by 1/{t} for the {t} ranks"}
    return res


def bench_tiny_mlp(ctx):
    """The tiny float32 MLP block (hidden 256, intermediate 1024, t=2, 4 tokens): a correctness
    configuration whose time is launch-bound; reported for completeness."""
    torch, tp, W, args = ctx.torch, ctx.tp, ctx.W, ctx.args
    wl = W.WORKLOADS[1]
    H, I, t = wl.hidden, wl.intermediate, wl.t
    M = args.tokens or wl.tokens[0]
    inp = W.mlp_inputs(1, H, I, M, "f32")
    desc = tp.make_desc(H, I, bytes_per_elem=4)
    plans = [tp.tp_shard_plan(desc, t, r) for r in range(t)]
    ranks = []
    for p in plans:
        b, n = p.inter_begin, p.inter_cols
        ranks.append({"w_gate": ctx.dev(ctx.phys(inp["w_gate"][:, b:b + n]), "f32"),
                      "w_up": ctx.dev(ctx.phys(inp["w_up"][:, b:b + n]), "f32"),
                      "w_down": ctx.dev(ctx.phys(inp["w_down"][b:b + n]), "f32")})
    x = ctx.dev(inp["x"], "f32")
    ws = tp.workspace(max(tp.tp_layer_workspace_bytes(desc, p, tp.TP_STAGE_MLP, M, tp.TP_F32) for p in plans))
    parts = [torch.empty(M, H, device="cuda") for _ in range(t)]
    out = torch.empty(M, H, device="cuda")

    def step(i):
        for r, p in enumerate(plans):
            tp.tp_layer_shard_forward(desc, p, tp.TP_STAGE_MLP, ranks[r], x, parts[r], ws=ws)
        tp.tp_partial_sum(parts, out)

    def shard(i):
        tp.tp_layer_shard_forward(desc, plans[i % t], tp.TP_STAGE_MLP, ranks[i % t], x, parts[i % t], ws=ws)

    for i in range(8):
        shard(i)
    sh = event_time_ms(torch, shard, 64)
    I_r = plans[0].inter_cols
    rank_bytes = 3 * I_r * H * 4 + M * H * 4 + M * H * 4
    total_ms = time_steps(ctx, step, 1)
    ms_step = total_ms / args.steps
    extra = {
        "per_rank": {"shard_us": sh[0] * 1e3, "bytes": rank_bytes},
        "roofline": roofline_hbm("gemv_kernel (float32 fma decode projections), both of one rank's MLP launches",
                                 f"tiny_mlp_m{M}", rank_bytes, *sh),
    }
    config = {"workload": f"tiny float32 MLP block, all t={t} rank shards + on-device sum (launch-bound)",
              "hidden": H, "intermediate": I, "t": t, "tokens": M}
    res = result(ctx, M * args.steps / (total_ms * 1e-3), "tokens/s", ms_step, config, extra)
    res["dtype"] = "f32"
    if not args.no_cpu:
        from oracle import layer as L
        from oracle import plan as OP
        od = OP.ModelDesc(hidden=H, intermediate=I)

        def rank(r):
            op = OP.rank_plan(od, t, r)
            b, c = op["inter_begin"], op["inter_cols"]
            return L.mlp_block(inp["x"], inp["w_gate"][:, b:b + c], inp["w_up"][:, b:b + c],
                               inp["w_down"][b:b + c])["y"]

        legs = time_legs(ctx, {"one_rank_shard": (lambda: rank(0), M),
                               "all_ranks_and_sum": (lambda: sum(rank(r) for r in range(t)), M),
                               "unsharded_block": (lambda: L.mlp_block(inp["x"], inp["w_gate"], inp["w_up"],
                                                                       inp["w_down"])["y"], M)},
                         "tokens_per_s", single_thread=("one_rank_shard", "all_ranks_and_sum"))
        res["cpu_baseline"] = {"value": legs["all_ranks_and_sum"]["tokens_per_s"], "unit": "tokens/s",
                               "cores": blas_threads(), "kind": "oracle",
                               "sample": f"float64 oracle (BLAS products), the whole step of {M} tokens; legs also "
                                         f"one rank and the unsharded block, and on one thread", "legs": legs,
                               "host": host_info()}
    return res


def bench_moe_prefill(ctx):
    """The Mixtral-8x7B-shaped MoE FFN prefill shard (t=2, 4096 tokens): each expert over the tokens
    routed to it. Throughput counts the routed flops (each token's top_k experts), not the dense ones."""
    torch, tp, W, args = ctx.torch, ctx.tp, ctx.W, ctx.args
    wl = W.WORKLOADS[9]
    H, I, t, E, k = wl.hidden, wl.intermediate, wl.t, W.MOE_EXPERTS, W.MOE_TOP_K
    M = args.tokens or wl.tokens[0]
    log(f"[bench] drawing {wl.name}")
    inp = W.moe_inputs(9, H, I, E, M, "bf16", progress=lambda e: log(f"[bench]   expert {e} drawn"))
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
    ws = tp.workspace(tp.tp_moe_workspace_bytes(M, H, E, k, cols, True))
    parts = [torch.empty(M, H, device="cuda") for _ in range(t)]
    out = torch.empty(M, H, dtype=torch.bfloat16, device="cuda")
    gates = torch.empty(M, E, device="cuda")

    def step(i, mk=None):
        for r in range(t):
            marked(mk, "moe", lambda: tp.tp_moe_shard_forward(ranks[r], x, parts[r], E, k, cols, eps=wl.eps, ws=ws))
        tp.tp_partial_sum(parts, out)

    # the routing, read back once for the routed flop count
    tp.tp_moe_shard_forward(ranks[0], x, parts[0], E, k, cols, eps=wl.eps, gates=gates, ws=ws)
    torch.cuda.synchronize()
    routed = int((gates > 0).sum().item())                      # = M * k
    fl_rank = 2.0 * routed * H * 2 * cols + 2.0 * routed * cols * H + 2.0 * M * H * E
    total_ms, mk = time_steps_eager(ctx, step)
    ms_step = total_ms / args.steps
    sh = mk.stats("moe")
    tf = fl_rank / (sh[0] * 1e-3) / 1e12
    log(f"[bench] MoE shard {sh[0] * 1e3:.1f} us ({tf:.0f} TFLOP/s routed) over {sh[3]} calls")
    tflops = t * fl_rank * args.steps / (total_ms * 1e-3) / 1e12
    extra = {
        "tokens_per_s": M * args.steps / (total_ms * 1e-3),
        "pct_mfma_peak": 100 * tflops / BF16_PEAK_TFLOPS,
        "per_rank": {"shard_us": sh[0] * 1e3, "routed_flops": fl_rank, "dense_flops": fl_rank * E / k,
                     "tokens_routed_per_expert": [int(v) for v in (gates > 0).sum(0).tolist()]},
        "roofline": {"kernel": "one rank's MoE shard call (router projection and gates, token lists, grouped "
                               "gate/up + SwiGLU GEMM, grouped down GEMM, slot sum)", "bound": "mfma",
                     "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS,
                     "traffic": counted_traffic(f"moe_prefill_m{M}"), "flops_per_launch": fl_rank,
                     "us_mean": sh[0] * 1e3, "us_median": sh[1] * 1e3, "us_min": sh[2] * 1e3,
                     "timed": f"every rank's call in the {args.steps} timed steps ({sh[3]} calls)"},
    }
    config = {"workload": f"Mixtral-8x7B-shaped MoE FFN prefill block, all t={t} rank shards + on-device sum, "
                          f"each expert over its routed tokens", "hidden": H, "intermediate": I, "experts": E,
              "top_k": k, "t": t, "tokens": M}
    res = result(ctx, tflops, "TFLOP/s", ms_step, config, extra)
    if not args.no_cpu:
        from oracle import layer as L
        from oracle import plan as OP
        n_tok = 64
        xs = inp["x"][:n_tok]
        gl = gates[:n_tok].cpu().numpy().astype(np.float64)
        op = OP.rank_plan(OP.ModelDesc(hidden=H, intermediate=I), t, 0)
        b, c = op["inter_begin"], op["inter_cols"]
        ex0 = [(g[:, b:b + c], u[:, b:b + c], d[b:b + c]) for g, u, d in inp["experts"]]
        log(f"[bench] CPU oracle for ~{args.cpu_seconds:.0f} s")
        n, el = repeat_for(args.cpu_seconds, lambda: L.moe_block(xs, inp["gamma"], inp["w_router"], ex0, k,
                                                                  gates=gl))
        sfl = fl_rank * n_tok / M
        res["cpu_baseline"] = {"value": n * sfl / el / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
                               "kind": "oracle",
                               "sample": f"{n} float64 passes (BLAS products) of rank 0's MoE shard over {n_tok} of "
                                         f"the {M} tokens with the GPU's routing, {el:.1f} s; counted on routed flops "
                                         f"(the oracle computes every expert densely, {E // k}x those)",
                               "host": host_info()}
    return res


if __name__ == "__main__":
    main()
