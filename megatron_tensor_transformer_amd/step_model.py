"""Per-token step time of a tensor-parallel decode, as a function of the degree t.

The model follows "Tensor parallel scaling curves", section *The scaling
math*: each of the t GPUs does 1/t of the matmul work and reads 1/t of the
weights, and every layer adds two all-reduces (one after the attention output
projection, one after the MLP down projection), each costing a per-call
latency plus a bandwidth term:

    T(t) = T_compute(1) / t + T_memory(1) / t + 2 L * T_allreduce(t)

The page's ring all-reduce moves 2 (t-1)/t of the message per GPU
(section *What tensor parallelism actually splits*). On an MI355X node every GPU has a
direct xGMI link to each of its seven peers, so a one-shot all-reduce (each
GPU reads its t-1 peers' partials over t-1 distinct links at once) moves one
message per link instead.

Pure host arithmetic: it predicts, it measures nothing. Inputs that the pages
do not give for MI355X (the per-call latency of an xGMI all-reduce) are
parameters, and the prediction labels them.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List


def allreduce_message_bytes(hidden: int, tokens: int = 1, bytes_per_elem: int = 2) -> int:
    """Bytes of one all-reduce message during decode: tokens x hidden activations."""
    return hidden * tokens * bytes_per_elem


def allreduce_calls(layers: int) -> int:
    """All-reduces per forward pass: two per layer (after W_o and after the down projection)."""
    return 2 * layers


@dataclass
class Interconnect:
    """One all-reduce's cost: a per-call latency plus bytes over per-link bandwidth."""
    latency_s: float
    link_bytes_per_s: float       # one direction of one link
    algorithm: str = "ring"       # "ring" (one link per GPU carries everything) or "one_shot" (t-1 links)

    def allreduce_s(self, t: int, message_bytes: float) -> float:
        if t <= 1:
            return 0.0
        if self.algorithm == "ring":
            moved = 2.0 * (t - 1) / t * message_bytes
        elif self.algorithm == "one_shot":
            moved = float(message_bytes)     # each peer's partial arrives over its own link, all at once
        else:
            raise ValueError(f"unknown all-reduce algorithm {self.algorithm!r}")
        return self.latency_s + moved / self.link_bytes_per_s


def step_time_s(t: int, t1_compute_s: float, t1_memory_s: float, layers: int, message_bytes: float,
                link: Interconnect) -> float:
    """T(t) = T_compute/t + T_memory/t + 2 L T_allreduce(t)."""
    if t < 1:
        raise ValueError("t must be >= 1")
    return t1_compute_s / t + t1_memory_s / t + allreduce_calls(layers) * link.allreduce_s(t, message_bytes)


def speedup(t: int, t1_compute_s: float, t1_memory_s: float, layers: int, message_bytes: float,
            link: Interconnect) -> float:
    base = step_time_s(1, t1_compute_s, t1_memory_s, layers, message_bytes, link)
    return base / step_time_s(t, t1_compute_s, t1_memory_s, layers, message_bytes, link)


# MI355X node figures: 7 xGMI links per GPU at about 153 GB/s each. The per-call
# latency of an all-reduce over xGMI is not given by the pages; the pages'
# NVLink range is 5-10 us, and the prediction uses its lower end unless told
# otherwise.
MI355X_XGMI_LINK_BYTES_PER_S = 153e9
DEFAULT_ALLREDUCE_LATENCY_S = 5e-6


def predict(layer_time_one_gpu_s: float, layers: int, hidden: int, tokens: int, max_t: int = 8,
            latency_s: float = DEFAULT_ALLREDUCE_LATENCY_S,
            link_bytes_per_s: float = MI355X_XGMI_LINK_BYTES_PER_S,
            algorithm: str = "one_shot") -> Dict[str, object]:
    """Predicted per-step time and speedup for t = 1..max_t.

    ``layer_time_one_gpu_s`` is one layer's decode time with all of its work on
    one GPU (for instance the measured time of all t rank shards of a layer
    run one after another on a single device). Decode is memory-bound, so
    the whole of it is counted as T_memory.
    """
    link = Interconnect(latency_s, link_bytes_per_s, algorithm)
    msg = allreduce_message_bytes(hidden, tokens)
    t1 = layer_time_one_gpu_s * layers
    rows: List[Dict[str, float]] = []
    for t in range(1, max_t + 1):
        st = step_time_s(t, 0.0, t1, layers, msg, link)
        rows.append({"t": t, "step_ms": st * 1e3, "speedup": t1 / st,
                     "allreduce_ms": allreduce_calls(layers) * link.allreduce_s(t, msg) * 1e3})
    return {"model": "T(t) = T_memory(1)/t + 2 L T_allreduce(t)", "layers": layers, "message_bytes": msg,
            "allreduce": algorithm, "allreduce_latency_us": latency_s * 1e6,
            "link_GBps": link_bytes_per_s / 1e9, "layer_time_one_gpu_us": layer_time_one_gpu_s * 1e6,
            "predicted": rows}
