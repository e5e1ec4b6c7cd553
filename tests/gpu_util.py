"""Helpers for the GPU parity tests: device buffers, host copies, comparisons."""

from __future__ import annotations

import sys

import numpy as np
import torch

import workloads as W
from expert_serving_amd import abi


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def workspace(shape) -> torch.Tensor:
    return torch.empty(abi.moe_workspace_size(shape), dtype=torch.uint8, device=dev())


def host(t):
    return W.to_numpy_raw(t)


def i32(n, fill=None):
    if fill is None:
        return torch.empty(n, dtype=torch.int32, device=dev())
    return torch.full((n,), fill, dtype=torch.int32, device=dev())


def f32(n):
    return torch.empty(n, dtype=torch.float32, device=dev())


def rms(a) -> float:
    a = np.asarray(a, np.float64)
    return float(np.sqrt((a ** 2).mean())) if a.size else 0.0


def assert_close_rms(got, ref, tol, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    r = rms(ref)
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    say(f"  {what}: max|err| = {err:.3e}, rms(ref) = {r:.3e}, ratio = {err / max(r, 1e-30):.3e} (tol {tol})")
    assert np.all(np.isfinite(got)), what
    assert err <= tol * r, f"{what}: max|err| {err} > {tol} * rms {r}"


def lazy_expert_copy(w: torch.Tensor, experts) -> np.ndarray:
    """Host copy of an [E, ...] weight holding only the listed experts (other
    pages are never touched, so never committed)."""
    E = w.shape[0]
    dt = np.uint16 if w.dtype == torch.bfloat16 else np.float32
    out = np.empty(tuple(w.shape), dt)
    for e in sorted(set(int(e) for e in experts)):
        assert 0 <= e < E
        out[e] = host(w[e])
    return out


def bf16_rel_tol():
    return 2e-2
