"""Shared plumbing for the GPU parity tests: device transfer, weight layout, the error metric.

The error metric is max |gpu - ref| / max |ref| per tensor, both sides in
float64; the tolerance is 1e-4 for float32 workloads and 2e-2 for bf16
workloads with float32 accumulation.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def tdtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Exact copy of storage-rounded float32 values to the device in the storage dtype."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(tdtype(dtype)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def phys(w_logical: np.ndarray) -> np.ndarray:
    """Logical [in, out] weight block to the ABI's physical [out, in] layout."""
    return np.ascontiguousarray(np.asarray(w_logical).T)


def relerr(gpu, ref) -> float:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    s = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / (s if s > 0 else 1.0))


def check(name: str, gpu, ref, tol: float):
    e = relerr(gpu, ref)
    say(f"  {name}: err {e:.3e} (tol {tol:.0e})")
    assert np.all(np.isfinite(np.asarray(gpu, np.float64))), f"{name}: non-finite output"
    assert e <= tol, f"{name}: err {e:.3e} > {tol:.0e}"
    return e
