"""The tensor-parallel step-time model against the arithmetic "Tensor parallel
scaling curves" prints in *The scaling math* and *What tensor parallelism actually splits*
(CPU only)."""
import math

import pytest

from megatron_tensor_transformer_amd import step_model as M


def test_message_and_call_counts():
    # 8192 hidden x 2 bytes = 16 KB per decode all-reduce; 80 layers -> 160 calls
    assert M.allreduce_message_bytes(8192) == 16384
    assert M.allreduce_calls(80) == 160


def test_page_example_tp2():
    # 160 calls x 8 us ~ 1.3 ms; 30 ms at TP=1 -> 15 ms + ~1.3 ms = 16.3 ms -> 1.84x
    link = M.Interconnect(latency_s=8e-6, link_bytes_per_s=float("inf"))
    msg = M.allreduce_message_bytes(8192)
    comm = M.allreduce_calls(80) * link.allreduce_s(2, msg)
    assert comm == pytest.approx(1.28e-3, rel=1e-12)
    t2 = M.step_time_s(2, 0.0, 30e-3, 80, msg, link)
    assert t2 == pytest.approx(16.28e-3, rel=1e-12)
    assert abs(t2 - 16.3e-3) < 0.05e-3
    assert M.speedup(2, 0.0, 30e-3, 80, msg, link) == pytest.approx(1.84, abs=5e-3)


def test_ring_bandwidth_term():
    # a ring moves 2 (N-1)/N of the message per GPU
    link = M.Interconnect(latency_s=0.0, link_bytes_per_s=1.0)
    for n in range(2, 9):
        assert link.allreduce_s(n, 1000.0) == pytest.approx(2.0 * (n - 1) / n * 1000.0)
    assert link.allreduce_s(1, 1000.0) == 0.0


def test_one_shot_moves_one_message_per_link():
    link = M.Interconnect(latency_s=1e-6, link_bytes_per_s=1e9, algorithm="one_shot")
    assert link.allreduce_s(8, 1e6) == pytest.approx(1e-6 + 1e-3)
    with pytest.raises(ValueError):
        M.Interconnect(0.0, 1.0, "tree").allreduce_s(2, 1.0)


def test_perfect_scaling_without_communication():
    link = M.Interconnect(latency_s=0.0, link_bytes_per_s=float("inf"))
    for t in range(1, 9):
        assert M.speedup(t, 2e-3, 6e-3, 80, 16384, link) == pytest.approx(t)


def test_latency_bends_the_curve():
    # a fixed per-call latency makes the speedup fall further below t as t grows
    link = M.Interconnect(latency_s=8e-6, link_bytes_per_s=450e9)
    eff = [M.speedup(t, 0.0, 30e-3, 80, 16384, link) / t for t in range(1, 9)]
    assert eff[0] == pytest.approx(1.0)
    assert all(a > b for a, b in zip(eff[1:], eff[2:]))


def test_predict_table():
    p = M.predict(layer_time_one_gpu_s=667e-6, layers=80, hidden=8192, tokens=16)
    rows = p["predicted"]
    assert [r["t"] for r in rows] == list(range(1, 9))
    assert rows[0]["speedup"] == pytest.approx(1.0)
    assert rows[0]["allreduce_ms"] == 0.0
    assert p["message_bytes"] == 16 * 8192 * 2
    assert all(math.isfinite(r["step_ms"]) and 0 < r["speedup"] <= r["t"] for r in rows)
