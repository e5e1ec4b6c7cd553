"""GPU parity of the MXFP8 expert path through the C ABI against the CPU oracle.

MXFP8 is the OCP Microscaling format (E4M3 elements, one E8M0 scale per 32
consecutive elements along the reduction axis); the pages serve FP8 experts
with the router kept in higher precision ("LLM MoE Expert Parallel production
practice", deployment examples; "Expert parallelism for MoE serving", FAQ).

* Quantiser: codes and scales bit-exact (the scale is a function of the block
  maximum's exponent field; the element rounding is IEEE nearest-even on an
  exactly scaled value, so there is one right answer).
* Grouped FFN and layer: both sides quantise x and the weights from the same
  bf16 values (bit-exact, checked above), so the operands are identical.  The
  GPU sums the products in fp32 in the MFMA's order and the oracle in fp64;
  each side then rounds its own h to E4M3, and where h lies within that
  summation difference of a rounding boundary the two keep neighbouring codes
  -- both correct roundings.  The check (tests/mx_check.py) requires the
  difference to be explained by such flips at near-ties (each a single E4M3
  step of one h element, seen through the down weights) plus a remainder
  below 1e-3 of the output RMS; it also reports max|err|/RMS.  The distance
  of the MXFP8 result from the bf16 oracle (the quantisation error itself) is
  printed as context, not compared.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from expert_serving_amd import abi

from gpu_util import dev, host, i32, lazy_expert_copy, rms, say, tile_cover_tokens
from mx_check import check_flips
from test_gpu_layer import check_routing

pytestmark = pytest.mark.gpu


def scales_to_rows(sc, rows, K, stride):
    """GPU scale layout (32-bit words of four block scales, group-major with
    the given row stride) -> [rows][K/32] bytes, the oracle's layout."""
    a = sc.cpu().numpy()[: (K // 128) * stride * 4].reshape(K // 128, stride, 4)
    return np.ascontiguousarray(a[:, :rows, :].transpose(1, 0, 2).reshape(rows, K // 32))


def gpu_quant(t, stride=None):
    K = t.shape[-1]
    rows = t.numel() // K
    codes, sc = abi.quantize_mxfp8(t, scale_stride=stride)
    torch.cuda.synchronize()
    return codes.cpu().numpy().reshape(rows, K), scales_to_rows(sc, rows, K, rows if stride is None else stride)


def wide_range(rng, rows, cols):
    a = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-20, 20, (rows, 1)))
    a *= np.exp2(rng.integers(-12, 1, (rows, cols)))
    a = a.astype(np.float32)
    a[0, :32] = 0.0                      # all-zero block
    a[1, :32] = 0.0
    a[1, 5] = 4.0                        # block maximum exactly a power of two
    a[1, 6] = -3.999
    a[2, :32] = 1.0
    a[2, 3] = 1.99                       # saturates to 448 after scaling
    a[3, 32:64] = -1e-3
    a[3, 40] = -1e-30                    # rounds to a signed zero
    return a


@pytest.mark.parametrize("src", ["f32", "bf16"])
@pytest.mark.parametrize("rows,cols", [(7, 128), (33, 640), (5, 1152)])
def test_quantize_bit_exact(src, rows, cols):
    say(f"mx quantise {src} {rows}x{cols}")
    a = wide_range(np.random.default_rng(rows * cols), rows, cols)
    t = torch.from_numpy(a)
    if src == "bf16":
        t = t.to(torch.bfloat16)
    ref_c, ref_s = oracle.mxfp8_quantize(W.to_numpy_raw(t))
    got_c, got_s = gpu_quant(t.to(dev()))
    assert np.array_equal(got_s, ref_s), np.argwhere(got_s != ref_s)[:5]
    bad = np.argwhere(got_c != ref_c)
    assert len(bad) == 0, [(tuple(i), int(got_c[tuple(i)]), int(ref_c[tuple(i)])) for i in bad[:5]]


def test_quantize_scale_stride():
    # scales written with a stride larger than the row count leave the gap alone
    t = W.normal((40, 256), 1.0, W.DT_BF16, dev(), 77)
    codes = torch.empty(40, 256, dtype=torch.uint8, device=dev())
    sc = torch.full((2 * 64 * 4,), 0xEE, dtype=torch.uint8, device=dev())
    abi.moe_quantize_mxfp8(40, 256, abi.MOE_BF16, t, 64, codes, sc)
    torch.cuda.synchronize()
    s = sc.cpu().numpy().reshape(2, 64, 4)
    assert (s[:, 40:, :] == 0xEE).all()
    ref_c, ref_s = oracle.mxfp8_quantize(host(t))
    assert np.array_equal(scales_to_rows(sc, 40, 256, 64), ref_s)
    assert np.array_equal(codes.cpu().numpy(), ref_c)


def mx_weights_gpu(wg, wu, wd):
    return abi.mxfp8_ffn(wg, wu, wd)


def mx_weights_oracle(wg, wu, wd):
    return dict(gate=oracle.mxfp8_quantize(wg), up=oracle.mxfp8_quantize(wu), down=oracle.mxfp8_quantize(wd))


FFN_CASES = [
    # name, E, H, I, rows per expert, tokens*k (sets the tile plan)
    ("big_tiles", 4, 512, 384, [300, 0, 77, 129], 4096),
    ("small_tiles", 8, 1024, 640, [16, 3, 0, 40, 17, 1, 64, 9], 150),
    ("both_classes_skew", 16, 256, 256, None, 1600),
    ("one_stage_k", 2, 128, 128, [300, 45], 600),
    ("odd_k_stages", 2, 384, 640, [520, 260], 1024),
    # remainders past the last full 256-row tile on 64-row tiles (no small expert)
    ("big_tiles_with_tails", 3, 512, 384, [300, 257, 552], 4096),
    # two one-row experts: gate/up K split into parts, h re-quantised by the
    # reduction kernel
    ("two_rows_split_gate_up", 8, 1024, 512, [1, 0, 0, 0, 0, 0, 1, 0], 2),
]


@pytest.mark.parametrize("name,E,H,I,rows,slots", FFN_CASES, ids=[c[0] for c in FFN_CASES])
def test_grouped_ffn_mxfp8_parity(name, E, H, I, rows, slots):
    say(f"mx ffn case {name}")
    if rows is None:
        rng = np.random.default_rng(9)
        p = np.arange(1, E + 1, dtype=np.float64) ** -1.3
        rows = rng.multinomial(slots, p / p.sum()).tolist()
    R = sum(rows)
    offsets = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    shape = abi.make_shape(num_tokens=slots, hidden=H, num_experts=E, intermediate=I, top_k=1)
    x = W.normal((slots, H), 1.0, W.DT_BF16, dev(), 31)
    wg = W.normal((E, I, H), H ** -0.5, W.DT_BF16, dev(), 32)
    wu = W.normal((E, I, H), H ** -0.5, W.DT_BF16, dev(), 33)
    wd = W.normal((E, H, I), I ** -0.5, W.DT_BF16, dev(), 34)
    mw = mx_weights_gpu(wg, wu, wd)
    xq, xs = abi.quantize_mxfp8(x)
    y = torch.full((slots, H), float("nan"), dtype=torch.float32, device=dev())
    ws = torch.empty(abi.moe_workspace_size_mxfp8(shape), dtype=torch.uint8, device=dev())
    abi.moe_grouped_ffn_mxfp8(shape, xq, xs, slots, torch.from_numpy(offsets).to(dev()), mw, y, ws)
    torch.cuda.synchronize()
    assert abi.moe_read_device_flags(ws) == 0
    ow = mx_weights_oracle(host(wg), host(wu), host(wd))
    oxq, oxs = oracle.mxfp8_quantize(host(x)[:R])
    ref, h32 = oracle.grouped_ffn_mxfp8(oxq, oxs, offsets, ow["gate"], ow["up"], ow["down"], return_h=True)
    got = y[:R].cpu().numpy()
    assert np.all(np.isfinite(got))
    r_ref = rms(ref)
    e_of = np.searchsorted(offsets, np.arange(R), side="right") - 1
    flips, rem = 0, 0.0
    for r in range(R):
        down_e = (ow["down"][0][e_of[r]], ow["down"][1][e_of[r]])
        f, m = check_flips(got[r].astype(np.float64) - ref[r], [(1.0, down_e, h32[r])], r_ref,
                           f"{name} row {r}")
        flips, rem = flips + f, max(rem, m)
    say(f"  {name}: {R} rows, {flips} rounding flips of h, remainder {rem / r_ref:.2e} * rms, "
        f"max|err|/rms {np.abs(got - ref).max() / r_ref:.2e}")
    if R < slots:
        assert torch.isnan(y[R:]).all()
    # context: distance from the unquantised bf16 FFN
    exact = oracle.grouped_ffn(host(x)[:R], offsets, host(wg), host(wu), host(wd))
    say(f"  quantisation error vs bf16 FFN: max|d|/rms = "
        f"{np.abs(y[:R].cpu().numpy() - exact).max() / rms(exact):.3e}")


def gpu_layer_mx(cfg, inp, mw, mws):
    T, E, k, H = cfg.tokens, cfg.experts, cfg.top_k, cfg.hidden
    shape = abi.make_shape(cfg)
    ws = torch.empty(abi.moe_workspace_size_mxfp8(shape), dtype=torch.uint8, device=dev())
    out = torch.empty(T, H, dtype=torch.float32, device=dev())
    dbg = dict(logits=torch.empty(T, E, dtype=torch.float32, device=dev()), topk_ids=i32(T * k),
               topk_gates=torch.empty(T * k, dtype=torch.float32, device=dev()), expert_counts=i32(E),
               expert_offsets=i32(E + 1), row_of_slot=i32(T * k), num_dropped=i32(1), row_token=i32(T * k))
    abi.moe_layer_forward_mxfp8(shape, inp["x"], inp["w_router"], inp["bias"], inp["k_per_token"], mw, mws,
                                out, dbg, ws)
    flags = abi.moe_read_device_flags(ws)
    res = {key: v.cpu().numpy() for key, v in dbg.items()}
    res["ids"] = res.pop("topk_ids").reshape(T, k)
    res["gates"] = res.pop("topk_gates").reshape(T, k)
    res["row_of_slot"] = res["row_of_slot"].reshape(T, k)
    res["num_dropped"] = int(res["num_dropped"][0])
    res["out"] = out.cpu().numpy()
    res["flags"] = flags
    return res


def compare_layer_mx(cfg, inp, sample=None, tiles=False, per_run=1):
    """Routing and dispatch bit-exact on every token (the oracle routes on
    the GPU's logits, as in test_gpu_layer.py); outputs of `sample` (None:
    all tokens), plus with `tiles` the tokens that put per_run compared rows
    into every 32-row run of every expert's rows (so every row tile of 64 or
    more rows has at least two), checked for rounding flips."""
    T = cfg.tokens
    say(f"mx layer {cfg.name}: T={T} H={cfg.hidden} E={cfg.experts} k={cfg.top_k} I={cfg.inter}")
    mw = mx_weights_gpu(inp["w_gate"], inp["w_up"], inp["w_down"])
    mws = mx_weights_gpu(inp["ws_gate"], inp["ws_up"], inp["ws_down"]) if cfg.shared_inter else None
    g = gpu_layer_mx(cfg, inp, mw, mws)
    assert g["flags"] == 0
    x_h, wr_h, b_h, kpt_h = host(inp["x"]), host(inp["w_router"]), host(inp["bias"]), host(inp["k_per_token"])
    d = check_routing(cfg, g, inp)
    ids_o = g["ids"]
    tokens = np.arange(T, dtype=np.int32) if sample is None else np.asarray(sample, np.int32)
    if tiles:
        cover, runs, covered = tile_cover_tokens(d["offsets"], d["row_token"], d["row_of_slot"], per_block=per_run)
        assert covered == runs
        say(f"  32-row runs of expert rows covered ({per_run} row each): {covered} of {runs} "
            f"(by {len(cover)} tokens)")
        tokens = np.union1d(tokens, cover).astype(np.int32)
    used = sorted(set(int(e) for e in ids_o[tokens].reshape(-1) if e >= 0))
    say(f"  quantising the weights of {len(used)} experts (oracle) ...")
    wq = {}
    for key, name in (("w_gate", "gate"), ("w_up", "up"), ("w_down", "down")):
        wl = lazy_expert_copy(inp[key], used)
        c = np.zeros(wl.shape, np.uint8)
        s = np.zeros(wl.shape[:-1] + (wl.shape[-1] // 32,), np.uint8)
        for e in used:
            c[e], s[e] = oracle.mxfp8_quantize(wl[e])
        wq[name] = (c, s)
    shared = None
    if cfg.shared_inter:
        shared = {n: oracle.mxfp8_quantize(host(inp[key]))
                  for key, n in (("ws_gate", "gate"), ("ws_up", "up"), ("ws_down", "down"))}
    say(f"  oracle layer on {len(tokens)} tokens ...")
    ref = oracle.layer_forward_mxfp8(x_h, wr_h, wq, cfg.top_k, b_h, kpt_h, cfg.score, cfg.renormalize,
                                     cfg.routed_scale, cfg.num_groups, cfg.topk_groups, cfg.group_topn,
                                     cfg.capacity_factor, shared, tokens=tokens, logits=g["logits"])
    assert np.array_equal(ref["ids"], ids_o)
    got = g["out"][tokens]
    assert np.all(np.isfinite(got))
    # output scale of the tokens that receive any expert output (with capacity
    # dropping, fully dropped tokens would otherwise shrink it)
    served = (ref["ros_c"] >= 0).any(1) | bool(cfg.shared_inter)
    r_ref = rms(ref["out"][served]) if served.any() else 1.0
    flips, rem = 0, 0.0
    for ti, t in enumerate(tokens):
        parts = [(float(ref["gates"][t, j]), (wq["down"][0][ids_o[t, j]], wq["down"][1][ids_o[t, j]]),
                  ref["h"][ref["ros_c"][ti, j]]) for j in range(cfg.top_k) if ref["ros_c"][ti, j] >= 0]
        if cfg.shared_inter:
            parts.append((1.0, shared["down"], ref["h_shared"][ti]))
        f, m = check_flips(got[ti].astype(np.float64) - ref["out"][ti], parts, r_ref, f"{cfg.name} token {t}")
        flips, rem = flips + f, max(rem, m)
        if ti % 200 == 199:
            say(f"  ... {ti + 1} of {len(tokens)} tokens checked")
    say(f"  {cfg.name}: {len(tokens)} tokens, {flips} rounding flips of h, remainder {rem / r_ref:.2e} * rms, "
        f"max|err|/rms {np.abs(got - ref['out']).max() / r_ref:.2e}")


LAYER_CASES = [
    ("mixtral_prefill", 32),
    ("mixtral_decode", None),   # all 64 tokens run; 24 of them are compared
    ("deepseek_v3", 24),
    ("qwen3_skewed", 256),
]


@pytest.mark.parametrize("name,T", LAYER_CASES, ids=[f"{c[0]}-T{c[1]}" for c in LAYER_CASES])
def test_layer_mxfp8_parity(name, T):
    cfg = W.CONFIGS[name]
    if T is not None:
        cfg = cfg.with_tokens(T)
    inp = W.make_layer_inputs(cfg, dev(), salt=1)
    compare_layer_mx(cfg, inp, sample=sample_tokens(cfg.tokens, 21) if name == "mixtral_decode" else None)


def sample_tokens(T, n, seed=0):
    rng = np.random.default_rng(seed)
    s = set([0, 1, T - 1]) | set(rng.choice(T, size=n, replace=False).tolist())
    return np.array(sorted(s), np.int32)


@pytest.mark.parametrize("name,n", [("mixtral_prefill", 12), ("deepseek_v3", 6), ("qwen3_skewed", 64)])
def test_layer_mxfp8_full_size_every_tile(name, n):
    """Full workload sizes: outputs of a random sample plus the tokens that
    cover every row tile of both classes."""
    cfg = W.CONFIGS[name]
    inp = W.make_layer_inputs(cfg, dev())
    compare_layer_mx(cfg, inp, sample=sample_tokens(cfg.tokens, n), tiles=True)


def test_layer_mxfp8_shared_mid_tiles_and_determinism():
    # 512 tokens: the shared expert runs on 128-row tiles
    cfg = W.CONFIGS["deepseek_v3"].with_tokens(512)
    inp = W.make_layer_inputs(cfg, dev(), salt=3)
    compare_layer_mx(cfg, inp, sample=sample_tokens(cfg.tokens, 5, seed=1))
    mw = mx_weights_gpu(inp["w_gate"], inp["w_up"], inp["w_down"])
    mws = mx_weights_gpu(inp["ws_gate"], inp["ws_up"], inp["ws_down"])
    a = gpu_layer_mx(cfg, inp, mw, mws)["out"]
    b = gpu_layer_mx(cfg, inp, mw, mws)["out"]
    assert np.array_equal(a, b)


def test_mxfp8_argument_errors():
    shape = abi.make_shape(num_tokens=8, hidden=192, num_experts=2, intermediate=128, top_k=1)
    with pytest.raises(abi.MoeError) as e:
        abi.moe_workspace_size_mxfp8(shape)
    assert e.value.status == abi.MOE_ERR_UNSUPPORTED
    shape = abi.make_shape(num_tokens=8, hidden=256, num_experts=2, intermediate=128, top_k=1,
                           act_dtype=abi.MOE_F32)
    with pytest.raises(abi.MoeError) as e:
        abi.moe_workspace_size_mxfp8(shape)
    assert e.value.status == abi.MOE_ERR_UNSUPPORTED
