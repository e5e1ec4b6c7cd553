"""GPU parity of the whole layer (moe_layer_forward, S1-S10) through the C ABI
against the CPU oracle, on every workload shape.

* Router logits: GPU and oracle both round to fp32 but sum in different
  orders; they must agree within 1e-5 * RMS (their own assertion).
* Routing, counts, offsets, row_of_slot, row_token and drops: the oracle
  routes on the GPU's own fp32 logits (routing is a function of those values
  alone), and every integer output must then match bit for bit on every
  token; gates within 1e-6 relative.  No token is exempt.
* Output: the oracle's layer routed on the same logits; max|err| <= 2e-2 *
  RMS(oracle output) over the compared tokens (bf16 inputs, fp32
  accumulation, h rounded to fp16); fp32 layers 1e-4.  Compared tokens are
  all tokens, or at the full workload sizes a set chosen from the permutation
  so that every 32-row run of every expert's rows -- hence every row tile of
  every class the grouped GEMMs launch, tails included -- has compared rows.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from expert_serving_amd import abi

from gpu_util import assert_close_rms, dev, host, i32, lazy_expert_copy, say, tile_cover_tokens, workspace

pytestmark = pytest.mark.gpu


def gpu_layer(cfg, inp):
    T, E, k, H = cfg.tokens, cfg.experts, cfg.top_k, cfg.hidden
    shape = abi.make_shape(cfg)
    ws = workspace(shape)
    out = torch.empty(T, H, dtype=torch.float32, device=dev())
    dbg = dict(logits=torch.empty(T, E, dtype=torch.float32, device=dev()), topk_ids=i32(T * k),
               topk_gates=torch.empty(T * k, dtype=torch.float32, device=dev()), expert_counts=i32(E),
               expert_offsets=i32(E + 1), row_of_slot=i32(T * k), num_dropped=i32(1), row_token=i32(T * k))
    abi.moe_layer_forward(shape, inp["x"], inp["w_router"], inp["bias"], inp["k_per_token"], inp["w_gate"],
                          inp["w_up"], inp["w_down"], inp["ws_gate"], inp["ws_up"], inp["ws_down"], out, dbg, ws)
    flags = abi.moe_read_device_flags(ws)
    res = {key: v.cpu().numpy() for key, v in dbg.items()}
    res["ids"] = res.pop("topk_ids").reshape(T, k)
    res["gates"] = res.pop("topk_gates").reshape(T, k)
    res["row_of_slot"] = res["row_of_slot"].reshape(T, k)
    res["num_dropped"] = int(res["num_dropped"][0])
    res["out"] = out
    res["flags"] = flags
    return res


def oracle_inputs(cfg, inp, tokens, ids_for_experts=None):
    """Host copies for the oracle; expert weights copied only where used."""
    d = {key: host(v) for key, v in inp.items() if key not in ("w_gate", "w_up", "w_down")}
    used = range(cfg.experts) if ids_for_experts is None else \
        sorted(set(int(e) for e in ids_for_experts[tokens].reshape(-1) if e >= 0))
    for key in ("w_gate", "w_up", "w_down"):
        d[key] = lazy_expert_copy(inp[key], used)
    return d


def check_routing(cfg, g, inp):
    """The GPU's logits against the oracle's own, then every routing and
    dispatch output against the oracle run on the GPU's logits: bit-exact on
    every token.  Returns the oracle's dispatch."""
    T = cfg.tokens
    x_h, wr_h, b_h, kpt_h = host(inp["x"]), host(inp["w_router"]), host(inp["bias"]), host(inp["k_per_token"])
    lo = oracle.router_logits(x_h, wr_h, b_h)
    assert_close_rms(g["logits"], lo, 1e-5, "logits (GPU vs the oracle's own sums)")
    route_args = (cfg.top_k, kpt_h, cfg.score, cfg.renormalize, cfg.routed_scale, cfg.num_groups,
                  cfg.topk_groups, cfg.group_topn)
    ids_o, gates_o = oracle.route(g["logits"], *route_args)
    bad = np.nonzero((g["ids"] != ids_o).any(1))[0]
    assert len(bad) == 0, f"{len(bad)} tokens route differently on the same logits, first {bad[:5]}: " \
                          f"gpu {g['ids'][bad[0]]} oracle {ids_o[bad[0]]}"
    np.testing.assert_allclose(g["gates"], gates_o, rtol=1e-6, atol=0)
    d = oracle.dispatch(ids_o, cfg.experts, cfg.capacity_factor)
    assert np.array_equal(g["expert_counts"], d["counts"])
    assert np.array_equal(g["expert_offsets"], d["offsets"])
    assert np.array_equal(g["row_of_slot"], d["row_of_slot"])
    assert np.array_equal(g["row_token"][:d["R"]], d["row_token"][:d["R"]])
    assert g["num_dropped"] == d["num_dropped"]
    # context: tokens the oracle's own logits would route otherwise (near ties)
    ids_own, _ = oracle.route(lo, *route_args)
    n_own = int((ids_own != ids_o).any(1).sum())
    say(f"  routing exact on all {T} tokens; R={d['R']} dropped={d['num_dropped']} "
        f"max/mean load={d['counts'].max() / max(d['counts'].mean(), 1e-9):.2f}; "
        f"tokens routed otherwise on the oracle's own logits: {n_own}")
    return d


def compare_layer(cfg, inp, sample=None, tiles=False):
    """sample: tokens whose outputs are compared (None: all).  tiles: add the
    tokens that give every 32-row run of every expert's rows compared rows."""
    T = cfg.tokens
    say(f"layer {cfg.name}: T={T} H={cfg.hidden} E={cfg.experts} k={cfg.top_k} I={cfg.inter}")
    g = gpu_layer(cfg, inp)
    torch.cuda.synchronize()
    d = check_routing(cfg, g, inp)
    assert g["flags"] == 0
    tokens = np.arange(T, dtype=np.int32) if sample is None else np.asarray(sample, np.int32)
    if tiles:
        cover, runs, covered = tile_cover_tokens(d["offsets"], d["row_token"], d["row_of_slot"])
        assert covered == runs
        say(f"  32-row runs of expert rows covered: {covered} of {runs} (by {len(cover)} tokens)")
        tokens = np.union1d(tokens, cover).astype(np.int32)
    oi = oracle_inputs(cfg, inp, tokens, g["ids"])
    ref = oracle.layer_forward_cfg(cfg, oi, tokens=tokens, logits=g["logits"])
    assert np.array_equal(ref["ids"], g["ids"])
    got = g["out"].cpu().numpy()[tokens]
    tol = 2e-2 if cfg.dtype == W.DT_BF16 else 1e-4
    assert_close_rms(got, ref["out"], tol, f"{cfg.name} out[{len(tokens)} tokens]")
    return d


SMALL = [
    ("tiny_fp32", None),
    ("mixtral_prefill", 96),
    ("mixtral_decode", None),
    ("deepseek_v3", 48),
    ("qwen3_skewed", 160),
]


@pytest.mark.parametrize("name,T", SMALL, ids=[f"{s[0]}-T{s[1]}" for s in SMALL])
def test_layer_parity_all_tokens(name, T):
    cfg = W.CONFIGS[name]
    if T is not None:
        cfg = cfg.with_tokens(T)
    inp = W.make_layer_inputs(cfg, dev(), salt=1)
    compare_layer(cfg, inp)


def sample_tokens(T, n=48, seed=0):
    rng = np.random.default_rng(seed)
    s = set([0, 1, T - 1, T - 2]) | set(rng.choice(T, size=n, replace=False).tolist())
    return np.array(sorted(s), np.int32)


@pytest.mark.parametrize("name", ["mixtral_prefill", "qwen3_skewed"])
def test_layer_parity_full_size_all_tokens(name):
    """The Mixtral-shaped prefill (4096 tokens) and Qwen3-shaped (16384
    tokens) workloads at full size, every output token compared."""
    cfg = W.CONFIGS[name]
    inp = W.make_layer_inputs(cfg, dev())
    compare_layer(cfg, inp)


def test_layer_parity_full_size_deepseek_v3_every_tile():
    """The DeepSeek-V3-shaped workload at full size (8192 tokens, 65536 rows
    in both tile classes): outputs compared on tokens that cover every row
    tile, plus a random sample."""
    cfg = W.CONFIGS["deepseek_v3"]
    inp = W.make_layer_inputs(cfg, dev())
    compare_layer(cfg, inp, sample=sample_tokens(cfg.tokens), tiles=True)


def test_layer_parity_shared_expert_mid_tiles():
    # 512 tokens put the shared expert on 128-row tiles (the 8-wave 128x128 kernel)
    cfg = W.CONFIGS["deepseek_v3"].with_tokens(512)
    inp = W.make_layer_inputs(cfg, dev(), salt=3)
    compare_layer(cfg, inp, sample=sample_tokens(cfg.tokens, n=40, seed=1), tiles=True)


def test_layer_deterministic_and_bf16_output():
    cfg = W.CONFIGS["qwen3_skewed"].with_tokens(2048)
    inp = W.make_layer_inputs(cfg, dev(), salt=2)
    a = gpu_layer(cfg, inp)["out"].clone()
    b = gpu_layer(cfg, inp)["out"]
    assert torch.equal(a, b)
    shape = abi.make_shape(cfg, out_dtype=abi.MOE_BF16)
    ws = workspace(shape)
    ob = torch.empty(cfg.tokens, cfg.hidden, dtype=torch.bfloat16, device=dev())
    abi.moe_layer_forward(shape, inp["x"], inp["w_router"], inp["bias"], inp["k_per_token"], inp["w_gate"],
                          inp["w_up"], inp["w_down"], None, None, None, ob, None, ws)
    assert torch.equal(ob, a.to(torch.bfloat16))


# every down-projection kernel path: merged big/small launch with the shared
# expert on 128-row tiles (DeepSeek-V3-shaped, 512 and 2048 tokens), a K-split
# merged launch (Mixtral-shaped, 256 tokens), 8-wave 32 x 256 tiles with a
# decode K-split (Mixtral-shaped decode), 4-wave 32 x 128 tiles (Qwen3-shaped,
# I = 768), and the shared expert on 32-row tiles (DeepSeek-V3-shaped, 5 tokens)
W16_CASES = [("deepseek_v3", 512), ("deepseek_v3", 2048), ("mixtral_prefill", 256), ("mixtral_decode", 64),
             ("qwen3_skewed", 1024), ("deepseek_v3", 5)]


@pytest.mark.parametrize("name,T", W16_CASES, ids=[f"{c[0]}-T{c[1]}" for c in W16_CASES])
def test_layer_with_fp16_down_weights_is_identical(name, T):
    """Down weights converted once by moe_convert_bf16_to_f16 and a shape with
    down_dtype = MOE_F16 give the layer output bit for bit: the conversion is
    the one the down projection applies to bf16 weights inside every call."""
    cfg = W.CONFIGS[name].with_tokens(T)
    say(f"fp16 down weights {name} T={T}")
    inp = W.make_layer_inputs(cfg, dev(), salt=4)
    ref = gpu_layer(cfg, inp)["out"]
    wd16 = abi.to_f16_weights(inp["w_down"])
    wsd16 = abi.to_f16_weights(inp["ws_down"]) if cfg.shared_inter else None
    shape = abi.make_shape(cfg, down_dtype=abi.MOE_F16)
    ws = workspace(shape)
    out = torch.empty_like(ref)
    abi.moe_layer_forward(shape, inp["x"], inp["w_router"], inp["bias"], inp["k_per_token"], inp["w_gate"],
                          inp["w_up"], wd16, inp["ws_gate"], inp["ws_up"], wsd16, out, None, ws)
    torch.cuda.synchronize()
    assert abi.moe_read_device_flags(ws) == 0
    assert torch.equal(out, ref), f"max |diff| {float((out - ref).abs().max())}"


def test_fp16_weight_conversion():
    """moe_convert_bf16_to_f16 against torch's conversion: identical wherever
    fp16 holds the bf16 value exactly (|w| in [2^-14, 65504]); below that,
    within one fp16 subnormal step (rounded toward zero); odd lengths."""
    g = torch.Generator(device="cpu").manual_seed(3)
    w = (torch.randn(4097, generator=g) * torch.exp2(torch.randint(-30, 12, (4097,), generator=g).float()))
    w = w.to(torch.bfloat16).to(dev())
    got = torch.empty(w.shape, dtype=torch.float16, device=dev())
    abi.moe_convert_bf16_to_f16(w.numel(), w, got)
    torch.cuda.synchronize()
    ref = w.float().cpu()
    got = got.float().cpu()
    normal = (ref.abs() >= 2.0 ** -14) & (ref.abs() <= 65504)
    assert torch.equal(got[normal], ref[normal])
    small = ref.abs() < 2.0 ** -14
    assert ((got[small] - ref[small]).abs() < 2.0 ** -24).all()
    assert ((got[small].abs() <= ref[small].abs())).all()
