"""CPU float64 oracle for one GPU's shard of a Megatron-style tensor-parallel layer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this package. The HIP
library never links, imports or calls it, and nothing here imports the HIP
package: the two share only the seeded input generator in ``workloads``.

Modules:
  plan     integer shard planner and memory footprints
  layer    the unsharded layer, written as its textbook definition
  sharded  the per-rank decomposition and the sum of partials, written separately
  naive    pure-Python loops for tiny shapes, used to pin the numpy code

Everything floating point runs in float64 on the exact values the GPU receives
(inputs are rounded to bf16 or fp32 by ``workloads`` and upcast exactly).

Pins (tests marked "not gpu"): the KV-cache worked example and the weight
footprint printed on "Tensor Parallelism Fundamentals"; the per-rank shapes of
the measured workloads; column shards concatenating to, and row partials
summing to, the unsharded result; closed forms of SiLU and RMSNorm; special
cases of decode attention; brute-force loops on tiny shapes; and planted
mistakes that the pins must catch. Layer output values themselves are printed
nowhere on the pages, so they are pinned only by those properties.
"""
