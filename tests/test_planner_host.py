"""The library's launch planners, queried on the host through a small C++ probe
(tests/plan_probe.cpp, linked against libtpshard.so; no GPU call is made).

- Split-K decode projections that merge in-kernel (the v_dot2 kernel, and the
  8-wave matrix-core kernel when it splits K over workgroups) keep one
  completion counter per (row tile, m-block) of a launch: a launch must never
  use more counters than the workspace header holds, however many row tiles
  the output has or however many tokens the batch has. (The 4-wave
  matrix-core kernel's splits go to a merge kernel and use no counters.)
- The 8-wave matrix-core kernel takes two blocks of 16 tokens per weight fetch
  only where it does not split K over workgroups (its slices and counters are
  per token block), and the decode shapes of 17 to 64 tokens take it.
- The decode attention's split-KV scratch depends on kv_len in a way that is
  not monotone, so the layer workspace sizes it by a bound over every kv_len up
  to the cache capacity; the bound must cover each kv_len.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "megatron_tensor_transformer_amd")


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("probe") / "plan_probe")
    cmd = [gxx, "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(PKG, "csrc"), os.path.join(ROOT, "tests", "plan_probe.cpp"), "-o", exe,
           "-L", PKG, "-ltpshard", f"-Wl,-rpath,{PKG}", "-L/opt/rocm/lib", "-lamdhip64"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)

    def run(lines):
        r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True,
                           timeout=300)
        out = []
        for ln in r.stdout.splitlines():
            out.append({k: int(v) for k, v in (kv.split("=") for kv in ln.split())})
        assert len(out) == len(lines)
        return out
    return run


def test_split_k_counters_fit_the_header(probe):
    queries = []
    for bf in (0, 1):
        for epi in ((0, 1, 2, 3) if bf else (0, 1, 2)):
            for m in (1, 2, 3, 4, 5, 8, 16, 20, 40, 64):
                for K in (256, 1024, 4096, 8192, 8200, 17000):
                    for N in (8, 1000, 1280, 70000, 128256, 150000, 600000):
                        queries.append((m, K, N, bf, epi))
    plans = probe([f"gemv {m} {K} {N} {bf} {epi}" for m, K, N, bf, epi in queries])
    big = mfma_split = 0
    for q, p in zip(queries, plans):
        assert 1 <= p["tiles_per_launch"] <= p["n_tiles"], (q, p)
        assert 1 <= p["mb_per_launch"] <= p["mblocks"], (q, p)
        counted = p["splits"] > 1 and (not p["mfma"] or p["waves"] == 8)
        if counted:
            assert p["tiles_per_launch"] * p["mb_per_launch"] <= p["header_counters"], (q, p)
            mfma_split += p["mfma"]
        if p["splits"] > 1:
            # the scratch holds every slice of one launch
            assert p["ws_bytes"] >= p["tiles_per_launch"] * p["mb_per_launch"] * p["splits"] * p["mt"] * \
                p["rows_per_tile"] * 4, (q, p)
            big += p["n_tiles"] > p["header_counters"]
    assert big > 0      # the sweep reaches outputs with more row tiles than counters
    assert mfma_split > 0   # and matrix-core plans that split K


@pytest.mark.parametrize("batch,q_heads,kv_heads,head_dim,capacity", [
    (16, 8, 1, 128, 2176), (1, 8, 1, 128, 66000), (16, 8, 1, 128, 8192), (20, 8, 1, 128, 3000),
    (3, 4, 2, 64, 300), (40, 16, 2, 128, 1000), (2, 8, 8, 128, 9999)])
def test_attention_scratch_bound_covers_every_kv_len(probe, batch, q_heads, kv_heads, head_dim, capacity):
    (r,) = probe([f"attn {batch} {q_heads} {kv_heads} {head_dim} {capacity}"])
    assert r["max_ws"] <= r["bound"], r


def test_two_token_blocks_per_weight_fetch(probe):
    queries = []
    for epi in (0, 1, 2, 3):
        for m in (1, 2, 16, 17, 20, 32, 33, 40, 48, 64):
            for K in (136, 1024, 3584, 4096, 8192, 8200):
                for N in (64, 1000, 1280, 2100, 4096, 7168, 8192, 14336):
                    queries.append((m, K, N, epi))
    plans = probe([f"gemv {m} {K} {N} 1 {epi}" for m, K, N, epi in queries])
    paired = 0
    for q, p in zip(queries, plans):
        assert p["mbw"] in (1, 2), (q, p)
        if p["mbw"] == 2:
            assert p["mfma"] == 1 and p["waves"] == 8 and p["splits"] == 1 and p["mblocks"] >= 2, (q, p)
            assert p["mb_per_launch"] == p["mblocks"], (q, p)
            paired += 1
        if p["mblocks"] == 1:
            assert p["mbw"] == 1, (q, p)
    assert paired > 0
    # every (output, token) pair is covered exactly once: row tiles of out_per_tile outputs (the gate and up
    # rows of each output sit in one tile), launches of mb_per_launch token blocks, and in each launch z
    # groups of mbw blocks of 16 tokens
    for q, p in zip(queries, plans):
        m, K, N, epi = q
        opt, rows = p["out_per_tile"], p["rows_per_tile"]
        assert 1 <= opt <= (rows // 2 if epi == 2 else rows), (q, p)
        assert p["n_tiles"] == -(-N // opt), (q, p)
        seen = [0] * p["mblocks"]
        for mb0 in range(0, p["mblocks"], p["mb_per_launch"]):
            blocks = min(p["mb_per_launch"], p["mblocks"] - mb0)
            for z in range(-(-blocks // p["mbw"])):
                first = mb0 + z * p["mbw"]
                for b in range(p["mbw"]):
                    if first + b < min(mb0 + blocks, p["mblocks"]):
                        seen[first + b] += 1
        assert seen == [1] * p["mblocks"] and p["mblocks"] * p["mt"] >= m > (p["mblocks"] - 1) * p["mt"], (q, p)
    # the 70B layer's gate/up, down and W_o shards at t=8 and the Llama-3-8B MLP shard at t=4, 17-64 tokens
    shapes = [(8192, 3584, 2), (3584, 8192, 1), (1024, 8192, 1), (4096, 3584, 2), (3584, 4096, 1)]
    got = probe([f"gemv {m} {K} {N} 1 {epi}" for m in (17, 32, 40, 64) for K, N, epi in shapes])
    assert all(p["mbw"] == 2 for p in got), got
