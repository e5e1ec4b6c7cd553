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

import oracle
from gpu_util import assert_close_rms, dev, say, tile_cover_tokens
from test_gpu_layer import check_routing, compare_layer, gpu_layer, oracle_inputs
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
    (compare_layer if fmt == "bf16" else compare_layer_mx)(cfg, inp, sample=sample, tiles=True)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8"])
def test_layer_big_tiles_k_split_three(fmt):
    """Mixtral-shaped with 256 tokens: 32 down tiles of 256 rows (at an even
    load) would leave most compute units idle, so the down projection splits
    K = 14336 into three parts, which the combine adds."""
    cfg = W.CONFIGS["mixtral_prefill"].with_tokens(256)
    say(f"big tiles, K split in three {fmt}")
    inp = W.make_layer_inputs(cfg, dev(), salt=11)
    # bf16: every token; MXFP8: the tokens covering every row tile (each
    # K-split part contributes to every row)
    if fmt == "bf16":
        compare_layer(cfg, inp)
    else:
        compare_layer_mx(cfg, inp, sample=np.array([0, 255], np.int32), tiles=True)


def test_layer_skinny_tiles_with_k_split():
    """Experts and tails of at most four rows inside the interleaved launch,
    with the down projection's K split in three: Mixtral-shaped, 512 tokens,
    and a router bias that gives the experts about 443, 260, 24, 127, 164, 3,
    2 and 1 rows (260 = one 256-row tile and a 4-row tail).  Rows of at most
    four run on the vector-ALU tiles (1, 2 or 4 token rows), the rest on MFMA
    tiles; every token is compared."""
    cfg = W.CONFIGS["mixtral_prefill"].with_tokens(512)
    say("skinny tiles, K split in three")
    inp = W.make_layer_inputs(cfg, dev(), salt=17)
    inp["bias"] = torch.tensor([3.019, 1.876, 0.246, 1.336, 1.412, -0.888, -0.835, -1.424], dtype=torch.float32,
                               device=dev())
    d = compare_layer(cfg, inp)
    counts = d["counts"]
    few = [int(c) for c in counts if 1 <= c <= 4] + [int(c) % 256 for c in counts if c >= 256 and 1 <= c % 256 <= 4]
    say(f"  rows per expert {counts.tolist()}; groups of 1-4 rows: {few}")
    assert len(few) >= 3 and counts.max() >= 256


def routed_layer_inputs(cfg, second, salt=23):
    """Layer inputs whose routing is set by hand: the router reads hidden
    dims 0..E-1 only (w_router = 10 * identity there) and x[t, :E] = +4 on the
    token's experts and -4 elsewhere, so token t's top-2 is {0, second[t]}."""
    inp = W.make_layer_inputs(cfg, dev(), salt=salt)
    E = cfg.experts
    code = torch.full((cfg.tokens, E), -4.0)
    code[:, 0] = 4.0
    code[torch.arange(cfg.tokens), torch.as_tensor(second)] = 4.0
    inp["x"][:, :E] = code.to(inp["x"].dtype).to(dev())
    wr = torch.zeros(E, cfg.hidden)
    wr[:, :E] = 10.0 * torch.eye(E)
    inp["w_router"] = wr.to(inp["w_router"].dtype).to(dev())
    return inp


def test_layer_fp16_range_flags():
    """|h| or |y| past the fp16 range inside a bf16 layer call sets
    MOE_FLAG_H_RANGE or MOE_FLAG_Y_RANGE, from every kind of tile: an expert
    on one 256-row MFMA tile (256 rows, no tail), one on a 64-row MFMA tile
    (20 rows) and one on vector-ALU tiles (2 rows), in one interleaved launch.
    One expert's gate and up (or down) weights are scaled up per call (the
    down weights far enough that their fp16 copies saturate); with the plain
    weights no flag is set."""
    cfg = W.CONFIGS["mixtral_prefill"].replace(hidden=1024, inter=2048, tokens=279)
    second = np.full(cfg.tokens, 4)
    second[:2] = 1
    second[2:22] = 2
    second[22] = 3
    say("fp16 range flags")
    inp = routed_layer_inputs(cfg, second)
    g = gpu_layer(cfg, inp)
    counts = g["expert_counts"]
    assert counts.tolist() == [279, 2, 20, 1, 256, 0, 0, 0], counts
    assert g["flags"] == 0
    for e, kind in ((4, "256-row tile"), (2, "64-row tile"), (1, "vector-ALU tiles")):
        for which, scale, flag in (("gate_up", 300.0, abi.MOE_FLAG_H_RANGE), ("down", 1e7, abi.MOE_FLAG_Y_RANGE)):
            keys = ("w_gate", "w_up") if which == "gate_up" else ("w_down",)
            saved = {key: inp[key][e].clone() for key in keys}
            for key in keys:
                inp[key][e] *= scale
            flags = gpu_layer(cfg, inp)["flags"]
            for key in keys:
                inp[key][e] = saved[key]
            say(f"  expert {e} ({kind}), {which} x {scale:g}: flags {flags}")
            assert flags & flag, (e, which, flags)


def test_layer_large_batch_every_tile():
    """32 times the Mixtral-shaped prefill batch: 131072 tokens, 262144 routed
    rows (h 7.5 GB and y 4.3 GB of workspace): the index arithmetic far past
    the benchmark's sizes.  Routing, counts and permutation are compared on
    every token (bit-exact, as in test_gpu_layer.py); outputs on the tokens
    that put two compared rows into every 256-row run of every expert's rows.
    Every expert holds about 32768 rows here, so the grouped GEMMs cut them
    into 256-row tiles from the expert's first row, with a remainder of at
    most 64 rows on one small tile at the start of the last run: each tile is
    one run."""
    cfg = W.CONFIGS["mixtral_prefill"].with_tokens(131072)
    say(f"large batch: T={cfg.tokens}")
    inp = W.make_layer_inputs(cfg, dev(), salt=5)
    g = gpu_layer(cfg, inp)
    torch.cuda.synchronize()
    d = check_routing(cfg, g, inp)
    assert g["flags"] == 0
    assert d["counts"].min() >= 256
    cover, runs, covered = tile_cover_tokens(d["offsets"], d["row_token"], d["row_of_slot"], block=256)
    assert covered == runs
    rng = np.random.default_rng(6)
    tokens = np.union1d(cover, rng.choice(cfg.tokens, 10, replace=False)).astype(np.int32)
    say(f"  256-row runs covered: {covered} of {runs} by {len(cover)} tokens")
    oi = oracle_inputs(cfg, inp, tokens, g["ids"])
    ref = oracle.layer_forward_cfg(cfg, oi, tokens=tokens, logits=g["logits"])
    assert_close_rms(g["out"].cpu().numpy()[tokens], ref["out"], 2e-2, f"out[{len(tokens)} tokens]")


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
