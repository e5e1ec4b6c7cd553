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


def tile_cover_tokens(offsets, row_token, row_of_slot, block=32, per_block=2, seed=0):
    """Tokens whose kept rows put at least min(per_block, rows in the run)
    compared rows into every `block`-row run of every expert's row range
    [offsets[e], offsets[e+1]), runs counted from the expert's first row.

    The grouped GEMMs cut each expert's rows into tiles of 32, 64, 128 or 256
    rows starting at multiples of the tile height from the expert's first
    row (a big expert's tail tile starts after its last full 256-row tile),
    so with block = 32 every row tile of every class is a union of these
    runs and has compared rows.  K-split parts need nothing more: each split
    part contributes to every output row.

    Greedy: runs are visited in order; a run still short of rows takes, among
    the tokens of its rows (a seeded sample of at most 32), the one whose rows
    fill the most still-short runs.  Returns (sorted tokens, runs, runs
    covered)."""
    offsets = np.asarray(offsets, np.int64)
    row_token = np.asarray(row_token)
    ros = np.asarray(row_of_slot).reshape(len(row_of_slot), -1)
    E = len(offsets) - 1
    R = int(offsets[E])
    starts, ends = [], []
    for e in range(E):
        for j in range(int(offsets[e]), int(offsets[e + 1]), block):
            starts.append(j)
            ends.append(min(j + block, int(offsets[e + 1])))
    starts = np.asarray(starts, np.int64)
    ends = np.asarray(ends, np.int64)
    run_of_row = np.empty(R, np.int64)
    for b, (a, z) in enumerate(zip(starts, ends)):
        run_of_row[a:z] = b
    need = np.minimum(per_block, ends - starts)
    have = np.zeros(len(starts), np.int64)
    chosen = set()
    rng = np.random.default_rng(seed)

    def runs_of(t):
        return [run_of_row[r] for r in ros[t] if r >= 0]

    for b in range(len(starts)):
        while have[b] < need[b]:
            a, z = int(starts[b]), int(ends[b])
            rows = a + rng.permutation(z - a)[:32]
            best, gain = -1, -1
            for r in rows:
                t = int(row_token[r])
                if t in chosen:
                    continue
                gn = sum(1 for q in runs_of(t) if have[q] < need[q])
                if gn > gain:
                    best, gain = t, gn
            if best < 0:   # every sampled row's token is taken: take any row of the run
                free = [int(row_token[r]) for r in range(a, z) if int(row_token[r]) not in chosen]
                if not free:
                    break
                best = free[0]
            chosen.add(best)
            for q in runs_of(best):
                have[q] += 1
    covered = int((have >= need).sum())
    return np.array(sorted(chosen), np.int32), len(starts), covered
