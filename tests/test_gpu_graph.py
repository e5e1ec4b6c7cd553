"""The layer call under HIP graph capture: every launch of moe_layer_forward
goes on the caller's stream with no host synchronisation and no memset
nodes, so the whole call can be captured once and replayed.  Each replay,
with eager work and synchronisations between replays, must reproduce the
eager result bit for bit (the path is deterministic)."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from expert_serving_amd import abi

from gpu_util import assert_close_rms, dev, i32, say, tile_cover_tokens, workspace
from test_gpu_layer import check_routing, oracle_inputs

pytestmark = pytest.mark.gpu


# qwen3_skewed T=1024: sliced vector router; T=2048: MFMA router with K split in
# two; mixtral_decode: decode K-split down; deepseek_v3 T=1: split-K gate/up
# (routed and shared expert) and its SwiGLU reduction
@pytest.mark.parametrize("name,T", [("qwen3_skewed", 1024), ("qwen3_skewed", 2048), ("mixtral_decode", 64),
                                    ("deepseek_v3", 1)])
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


def test_one_graph_serves_every_k_mix():
    """Per-token k ("MoE-Prism: Disentangling Monolithic Experts...", the
    k-aware execution part: MoE graph segments specialised per k) is read on
    the device here, so one captured layer call serves any mix of k values:
    rewriting k_per_token in place between replays must give what an eager
    call with the new k gives, bit for bit, and the replay must match the
    oracle run with the rewritten k: routing, counts, offsets, permutation
    and drops bit-exact on every token, outputs within 2e-2 * RMS on a
    sample plus the tokens that cover every row tile."""
    cfg = W.CONFIGS["qwen3_skewed"].with_tokens(2048)
    say("graph capture qwen3_skewed T=2048, k rewritten between replays")
    inp = W.make_layer_inputs(cfg, dev(), salt=6)
    shape = abi.make_shape(cfg)
    ws = workspace(shape)
    T, E, kmax = cfg.tokens, cfg.experts, cfg.top_k
    out = torch.empty(T, cfg.hidden, dtype=torch.float32, device=dev())
    k = inp["k_per_token"]
    assert k is not None and k.dtype == torch.int32
    dbg = dict(logits=torch.empty(T, E, dtype=torch.float32, device=dev()), topk_ids=i32(T * kmax),
               topk_gates=torch.empty(T * kmax, dtype=torch.float32, device=dev()), expert_counts=i32(E),
               expert_offsets=i32(E + 1), row_of_slot=i32(T * kmax), num_dropped=i32(1),
               row_token=i32(T * kmax))

    def call():
        abi.moe_layer_forward(shape, inp["x"], inp["w_router"], inp["bias"], k, inp["w_gate"], inp["w_up"],
                              inp["w_down"], inp["ws_gate"], inp["ws_up"], inp["ws_down"], out, dbg, ws)

    def replayed():
        res = {key: v.cpu().numpy() for key, v in dbg.items()}
        res["ids"] = res.pop("topk_ids").reshape(T, kmax)
        res["gates"] = res.pop("topk_gates").reshape(T, kmax)
        res["row_of_slot"] = res["row_of_slot"].reshape(T, kmax)
        res["num_dropped"] = int(res["num_dropped"][0])
        return res

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()

    gen = torch.Generator().manual_seed(11)
    mixes = {
        "all k_max": torch.full((cfg.tokens,), cfg.top_k, dtype=torch.int32),
        "all 2": torch.full((cfg.tokens,), 2, dtype=torch.int32),
        "k in 1..k_max": torch.randint(1, cfg.top_k + 1, (cfg.tokens,), generator=gen, dtype=torch.int32),
        "sorted tiers": torch.sort(torch.tensor(cfg.k_choices, dtype=torch.int32)[
            torch.randint(0, len(cfg.k_choices), (cfg.tokens,), generator=gen)])[0].to(torch.int32),
    }
    for name, kk in mixes.items():
        k.copy_(kk.to(dev()))
        call()
        torch.cuda.synchronize()
        ref = out.clone()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay with k mix '{name}' differs from the eager call"
        assert abi.moe_read_device_flags(ws) == 0
        # the replay against the oracle with the rewritten k
        say(f"  k mix '{name}': sum of k_t = {int(kk.sum())}")
        r = replayed()
        d = check_routing(cfg, r, inp)
        cover, runs, covered = tile_cover_tokens(d["offsets"], d["row_token"], d["row_of_slot"])
        assert covered == runs
        tokens = np.union1d(cover, np.arange(0, T, 97)).astype(np.int32)
        oi = oracle_inputs(cfg, inp, tokens, r["ids"])
        o = oracle.layer_forward_cfg(cfg, oi, tokens=tokens, logits=r["logits"])
        assert_close_rms(out.cpu().numpy()[tokens], o["out"], 2e-2,
                         f"replay, k mix '{name}', out[{len(tokens)} tokens, {covered} of {runs} 32-row runs]")
