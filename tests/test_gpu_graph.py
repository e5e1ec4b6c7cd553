"""The layer call under HIP graph capture: every launch of moe_layer_forward
goes on the caller's stream with no host synchronisation and no memset
nodes, so the whole call can be captured once and replayed.  Each replay,
with eager work and synchronisations between replays, must reproduce the
eager result bit for bit (the path is deterministic)."""

import pytest
import torch

import workloads as W
from expert_serving_amd import abi

from gpu_util import dev, say, workspace

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T", [("qwen3_skewed", 1024), ("mixtral_decode", 64)])
def test_layer_graph_replay_matches_eager(name, T):
    cfg = W.CONFIGS[name].with_tokens(T)
    say(f"graph capture {name} T={T}")
    inp = W.make_layer_inputs(cfg, dev(), salt=5)
    shape = abi.make_shape(cfg)
    ws = workspace(shape)
    out = torch.empty(cfg.tokens, cfg.hidden, dtype=torch.float32, device=dev())

    def call():
        abi.moe_layer_forward(shape, inp["x"], inp["w_router"], inp["bias"], inp["k_per_token"], inp["w_gate"],
                              inp["w_up"], inp["w_down"], inp["ws_gate"], inp["ws_up"], inp["ws_down"], out, None, ws)

    call()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(4):
        out.fill_(float("nan"))
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager result"
        # eager work between replays
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
    assert abi.moe_read_device_flags(ws) == 0
