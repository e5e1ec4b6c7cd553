"""moe_layer_forward_noalloc (the layer with its workspace in the library's own
device array) against moe_layer_forward (caller workspace) through the C ABI.

Both run the same kernels, so every output must be bit-identical: the layer
output and the routing, counts, offsets, permutation and drops.  The calls
run back to back, each case smaller than the one before, so a later call
finds the array holding the previous call's contents.
"""

import numpy as np
import pytest
import torch

import workloads as W
from expert_serving_amd import abi

from gpu_util import dev, i32, say, workspace

pytestmark = pytest.mark.gpu

# (workload, tokens): largest first; the second and third calls are smaller
CASES = [("deepseek_v3", 64), ("deepseek_v3", 5), ("qwen3_skewed", 48), ("mixtral_decode", 16)]


def run(cfg, inp, noalloc):
    T, E, k, H = cfg.tokens, cfg.experts, cfg.top_k, cfg.hidden
    shape = abi.make_shape(cfg)
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device=dev())
    dbg = dict(logits=torch.empty(T, E, dtype=torch.float32, device=dev()), topk_ids=i32(T * k),
               topk_gates=torch.empty(T * k, dtype=torch.float32, device=dev()), expert_counts=i32(E),
               expert_offsets=i32(E + 1), row_of_slot=i32(T * k), num_dropped=i32(1))
    args = (shape, inp["x"], inp["w_router"], inp["bias"], inp["k_per_token"], inp["w_gate"], inp["w_up"],
            inp["w_down"], inp["ws_gate"], inp["ws_up"], inp["ws_down"], out, dbg)
    if noalloc:
        abi.moe_layer_forward_noalloc(*args)
    else:
        ws = workspace(shape)
        ws.fill_(0xA5)      # stale contents in the caller's workspace too
        abi.moe_layer_forward(*args, ws)
    torch.cuda.synchronize()
    res = {key: v.cpu() for key, v in dbg.items()}
    res["out"] = out.cpu()
    return res


def test_noalloc_matches_workspace_entry_point():
    for name, T in CASES:
        cfg = W.CONFIGS[name].with_tokens(T)
        shape = abi.make_shape(cfg)
        assert abi.moe_workspace_size(shape) <= abi.MOE_NOALLOC_SCRATCH_BYTES
        say(f"noalloc {name} T={T}: workspace {abi.moe_workspace_size(shape) / 2**20:.1f} MiB")
        inp = W.make_layer_inputs(cfg, dev(), salt=7)
        a = run(cfg, inp, noalloc=True)
        b = run(cfg, inp, noalloc=False)
        for key in b:
            assert torch.equal(a[key], b[key]), f"{name} T={T}: {key} differs"
        assert torch.isfinite(a["out"]).all()
        say(f"  identical; rows kept {int(a['expert_offsets'][-1])}, "
            f"rms(out) {float(a['out'].double().pow(2).mean().sqrt()):.3e}")


def test_noalloc_rejects_oversized_shape():
    cfg = W.CONFIGS["deepseek_v3"].with_tokens(1024)
    shape = abi.make_shape(cfg)
    assert abi.moe_workspace_size(shape) > abi.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.uint8, device=dev())
    with pytest.raises(abi.MoeError) as e:
        abi.moe_layer_forward_noalloc(shape, x, x, None, None, x, x, x, x, x, x, x, None)
    assert e.value.status == abi.MOE_ERR_WORKSPACE
