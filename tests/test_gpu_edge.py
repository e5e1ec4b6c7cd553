"""Edge cases of the layer through the C ABI, bf16 and MXFP8 experts: an empty
batch, a single token, one expert (the layer is then a dense SwiGLU FFN),
every expert selected (k = E, no renormalisation: the dense softmax
mixture), a capacity of one row per expert, and graph capture of the MXFP8
layer.  Comparisons as in test_gpu_layer.py (bf16) and test_gpu_mxfp8.py
(MXFP8)."""

import numpy as np
import pytest
import torch

import workloads as W
from expert_serving_amd import abi

from gpu_util import dev, say
from test_gpu_layer import compare_layer
from test_gpu_mxfp8 import compare_layer_mx

pytestmark = pytest.mark.gpu

EDGE = {
    # one expert, k = 1: the layer is one dense SwiGLU FFN with gate 1
    "one_expert": W.LayerConfig("one_expert", 300, 512, 1, 256, 1),
    # every expert selected without renormalisation: the dense softmax mixture
    "all_experts": W.LayerConfig("all_experts", 200, 512, 4, 256, 4, renormalize=0),
    # capacity ceil(1e-4 * 512 / 8) = 1: each expert keeps its first slot
    "capacity_one": W.LayerConfig("capacity_one", 256, 512, 8, 256, 2, capacity_factor=1e-4),
}


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8"])
@pytest.mark.parametrize("name", list(EDGE))
def test_layer_edge_shapes(name, fmt):
    cfg = EDGE[name]
    say(f"edge {name} {fmt}")
    inp = W.make_layer_inputs(cfg, dev(), salt=7)
    (compare_layer if fmt == "bf16" else compare_layer_mx)(cfg, inp)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8"])
@pytest.mark.parametrize("name", ["mixtral_prefill", "deepseek_v3"])
def test_layer_single_token(name, fmt):
    cfg = W.CONFIGS[name].with_tokens(1)
    say(f"single token {name} {fmt}")
    inp = W.make_layer_inputs(cfg, dev(), salt=8)
    (compare_layer if fmt == "bf16" else compare_layer_mx)(cfg, inp)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8"])
@pytest.mark.parametrize("name,T", [("mixtral_prefill", 3), ("deepseek_v3", 5), ("deepseek_v3", 2)])
def test_layer_few_tokens_split_gate_up(name, T, fmt):
    """A few tokens: the gate/up projection's K is split into parts (their
    weight-streaming tiles fill one or two rounds of the compute units
    poorly), the parts added by the SwiGLU reduction kernel."""
    cfg = W.CONFIGS[name].with_tokens(T)
    say(f"few tokens {name} T={T} {fmt}")
    inp = W.make_layer_inputs(cfg, dev(), salt=12)
    (compare_layer if fmt == "bf16" else compare_layer_mx)(cfg, inp)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8"])
def test_layer_interleaved_classes_with_shared_expert(fmt):
    """DeepSeek-V3-shaped with 2048 tokens (average load 64 rows, the
    smallest batch that interleaves both tile classes in one launch per
    projection), with the shared expert on 256-row tiles."""
    cfg = W.CONFIGS["deepseek_v3"].with_tokens(2048)
    say(f"interleaved classes with shared expert {fmt}")
    inp = W.make_layer_inputs(cfg, dev(), salt=10)
    rng = np.random.default_rng(3)
    sample = np.array(sorted(set([0, 2047]) | set(rng.choice(2048, 14, replace=False).tolist())), np.int32)
    (compare_layer if fmt == "bf16" else compare_layer_mx)(cfg, inp, sample=sample)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8"])
def test_layer_big_tiles_k_split_three(fmt):
    """Mixtral-shaped with 256 tokens: 32 down tiles of 256 rows (at an even
    load) would leave most compute units idle, so the down projection splits
    K = 14336 into three parts, which the combine adds."""
    cfg = W.CONFIGS["mixtral_prefill"].with_tokens(256)
    say(f"big tiles, K split in three {fmt}")
    inp = W.make_layer_inputs(cfg, dev(), salt=11)
    rng = np.random.default_rng(4)
    sample = np.array(sorted(set([0, 255]) | set(rng.choice(256, 14, replace=False).tolist())), np.int32)
    (compare_layer if fmt == "bf16" else compare_layer_mx)(cfg, inp, sample=sample)


def test_layer_large_batch_sampled():
    """32 times the Mixtral-shaped prefill batch: 131072 tokens, 262144 routed
    rows (h 7.5 GB and y 4.3 GB of workspace).  Routing, counts and
    permutation are compared on every token (near ties allowed as in
    test_gpu_layer.py), outputs on a sample: the index arithmetic far past
    the benchmark's sizes."""
    cfg = W.CONFIGS["mixtral_prefill"].with_tokens(131072)
    say(f"large batch: T={cfg.tokens}")
    inp = W.make_layer_inputs(cfg, dev(), salt=5)
    rng = np.random.default_rng(6)
    sample = np.array(sorted(set([0, cfg.tokens - 1]) | set(rng.choice(cfg.tokens, 10, replace=False).tolist())),
                      np.int32)
    compare_layer(cfg, inp, sample=sample)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8"])
def test_layer_empty_batch(fmt):
    """T = 0: the call succeeds, launches nothing and writes nothing."""
    cfg = W.CONFIGS["deepseek_v3"].with_tokens(0)
    shape = abi.make_shape(cfg)
    H = cfg.hidden
    say(f"empty batch {fmt}")
    dummy = torch.zeros(64, dtype=torch.float32, device=dev())  # any valid aligned pointer
    out = torch.full((4, H), 7.0, dtype=torch.float32, device=dev())
    if fmt == "bf16":
        ws = torch.empty(max(abi.moe_workspace_size(shape), 256), dtype=torch.uint8, device=dev())
        abi.moe_layer_forward(shape, dummy, dummy, dummy, None, dummy, dummy, dummy, dummy, dummy, dummy, out,
                              None, ws)
    else:
        ws = torch.empty(max(abi.moe_workspace_size_mxfp8(shape), 256), dtype=torch.uint8, device=dev())
        ffn = abi.MoeMxfp8Ffn(*([dummy.data_ptr()] * 6))
        abi.moe_layer_forward_mxfp8(shape, dummy, dummy, dummy, None, ffn, ffn, out, None, ws)
    torch.cuda.synchronize()
    assert (out == 7.0).all()


@pytest.mark.parametrize("name,T", [("mixtral_decode", 64), ("qwen3_skewed", 1024), ("deepseek_v3", 1)])
def test_mxfp8_layer_graph_replay_matches_eager(name, T):
    """The MXFP8 layer call captured once and replayed, with eager calls and
    synchronisations between replays, reproduces the eager result bit for bit."""
    cfg = W.CONFIGS[name].with_tokens(T)
    say(f"mxfp8 graph capture {name} T={T}")
    inp = W.make_layer_inputs(cfg, dev(), salt=9)
    mw = abi.mxfp8_ffn(inp["w_gate"], inp["w_up"], inp["w_down"])
    mws = abi.mxfp8_ffn(inp["ws_gate"], inp["ws_up"], inp["ws_down"]) if cfg.shared_inter else None
    shape = abi.make_shape(cfg)
    ws = torch.empty(abi.moe_workspace_size_mxfp8(shape), dtype=torch.uint8, device=dev())
    out = torch.empty(cfg.tokens, cfg.hidden, dtype=torch.float32, device=dev())

    def call():
        abi.moe_layer_forward_mxfp8(shape, inp["x"], inp["w_router"], inp["bias"], inp["k_per_token"], mw, mws,
                                    out, None, ws)

    call()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        out.fill_(float("nan"))
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager result"
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    assert abi.moe_read_device_flags(ws) == 0
