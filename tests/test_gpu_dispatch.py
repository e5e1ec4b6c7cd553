"""GPU parity of dispatch (S3 histogram, S4 capacity/offsets, S5 stable
permutation, S6 gather) through the C ABI against the CPU oracle: every
integer output bit-exact, the gathered rows bitwise equal."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from expert_serving_amd import abi

from gpu_util import dev, host, i32, say, workspace

pytestmark = pytest.mark.gpu

DISPATCH_CASES = [
    # name, T, E, k, cf, per-token k choices, zipf
    ("qwen_full", 16384, 128, 8, 1.25, (2, 4, 6, 8), 1.2),
    ("deepseek_full", 8192, 256, 8, 0.0, None, 1.1),
    ("mixtral_full_cap1", 4096, 8, 2, 1.0, None, 0.0),
    ("heavy_drop", 3000, 16, 4, 0.3, None, 0.8),
    ("capacity_one", 700, 10, 3, 1.0 / 32.0, None, 0.0),
    ("one_token", 1, 8, 2, 0.0, None, 0.0),
    ("ragged_tiles", 2049, 5, 3, 0.0, (1, 2, 3), 0.5),
    ("e512", 900, 512, 16, 0.0, None, 1.0),
    # all slots in one tile (the fused single-block path): drops with per-token k,
    # exactly one full tile, 512 experts, one expert
    ("single_tile_capacity", 300, 16, 3, 0.5, (1, 2, 3), 0.8),
    ("single_tile_full", 512, 8, 2, 0.0, None, 0.0),
    ("single_tile_e512", 60, 512, 16, 1.0, None, 1.0),
    ("single_tile_one_expert", 700, 1, 1, 0.0, None, 0.0),
]


def run_dispatch(T, E, k, cf, ids_np, x=None):
    shape = abi.make_shape(num_tokens=T, hidden=x.shape[1] if x is not None else 64, num_experts=E,
                           intermediate=64, top_k=k, capacity_factor=cf)
    ws = workspace(shape)
    ids = torch.from_numpy(ids_np.reshape(-1)).to(dev())
    counts, offsets = i32(E, -9), i32(E + 1, -9)
    ros, row_token, nd = i32(T * k, -9), i32(T * k, -9), i32(1, -9)
    x_perm = torch.empty(T * k, x.shape[1], dtype=x.dtype, device=dev()) if x is not None else None
    abi.moe_dispatch(shape, x, ids, counts, offsets, ros, row_token, nd, x_perm, ws)
    flags = abi.moe_read_device_flags(ws)
    return dict(counts=counts.cpu().numpy(), offsets=offsets.cpu().numpy(),
                row_of_slot=ros.cpu().numpy().reshape(T, k), row_token=row_token.cpu().numpy(),
                num_dropped=int(nd.cpu().numpy()[0]), x_perm=x_perm, flags=flags)


@pytest.mark.parametrize("name,T,E,k,cf,kch,zipf", DISPATCH_CASES, ids=[c[0] for c in DISPATCH_CASES])
def test_dispatch_parity(name, T, E, k, cf, kch, zipf):
    say(f"dispatch case {name}: T={T} E={E} k={k} cf={cf}")
    bias = W.log_zipf_bias(E, zipf) if zipf > 0 else None
    logits = W.make_logits(T, E, seed=T + E, bias=bias).numpy()
    kpt = W.make_k_per_token(T, kch, seed=5).numpy() if kch else None
    ids, _ = oracle.route(logits, k, kpt)
    ref = oracle.dispatch(ids, E, cf)
    x = W.normal((T, 128), 1.0, W.DT_BF16, dev(), 3)
    got = run_dispatch(T, E, k, cf, ids, x)
    assert np.array_equal(got["counts"], ref["counts"])
    assert np.array_equal(got["offsets"], ref["offsets"])
    assert np.array_equal(got["row_of_slot"], ref["row_of_slot"])
    R = ref["R"]
    assert np.array_equal(got["row_token"][:R], ref["row_token"][:R])
    assert got["num_dropped"] == ref["num_dropped"]
    assert got["flags"] == 0
    xp = host(got["x_perm"][:R])
    assert np.array_equal(xp, host(x)[ref["row_token"][:R]])
    say(f"  R={R} dropped={ref['num_dropped']} max/mean={ref['counts'].max() / max(ref['counts'].mean(), 1e-9):.2f}")


@pytest.mark.parametrize("T", [500, 300], ids=["tiled", "single_tile"])
def test_dispatch_invalid_ids_flagged_and_unused(T):
    E, k = 12, 3
    ids, _ = oracle.route(W.make_logits(T, E, seed=99).numpy(), k)
    ids = ids.copy()
    ids[5, 1] = E + 3
    ids[77, 0] = -5
    ids[T - 100, 2] = -1
    ref = oracle.dispatch(ids, E, 0.0)        # the oracle also skips ids outside [0, E)
    got = run_dispatch(T, E, k, 0.0, ids)
    assert got["flags"] == abi.MOE_FLAG_BAD_EXPERT
    assert np.array_equal(got["row_of_slot"], ref["row_of_slot"])
    assert np.array_equal(got["offsets"], ref["offsets"])
    assert got["row_of_slot"][5, 1] == -1 and got["row_of_slot"][77, 0] == -1


def test_dispatch_is_deterministic():
    T, E, k = 16384, 128, 8
    ids, _ = oracle.route(W.make_logits(T, E, seed=3, bias=W.log_zipf_bias(E, 1.2)).numpy(), k)
    a = run_dispatch(T, E, k, 1.25, ids)
    b = run_dispatch(T, E, k, 1.25, ids)
    for key in ("counts", "offsets", "row_of_slot", "row_token"):
        assert np.array_equal(a[key], b[key])
