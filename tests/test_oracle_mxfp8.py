"""Pins of the oracle's MXFP8 path (CPU only).

MXFP8 follows the OCP Microscaling Formats specification v1.0 (32-element
blocks along the reduction axis, one E8M0 power-of-two scale per block, E4M3
elements).  The pages ask for FP8 experts with the router kept in higher
precision ("LLM MoE Expert Parallel production practice", deployment
examples; "Expert parallelism for MoE serving", FAQ) and fix no scaling
granularity.  Each pin below checks the oracle against something other than
its own formulas: torch's float8_e4m3fn conversion (a library routine),
brute force over all codes, exact round trips, numpy's frexp, the element
error bound, and a float64 numpy evaluation of the FFN."""

import numpy as np
import pytest
import torch

import oracle


def torch_e4m3_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy().astype(np.float64)


def torch_e4m3_encode(v):
    """torch's float32 -> float8_e4m3fn conversion (round to nearest even),
    after saturating to +-448 (torch maps larger magnitudes to NaN)."""
    v = np.clip(np.asarray(v, np.float32), -448.0, 448.0)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_values_match_torch():
    codes = np.arange(256)
    ours = oracle.e4m3_value(codes)
    ref = torch_e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(codes[nan]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    # the positive finite codes are strictly increasing; largest 448, smallest 2^-9
    pos = ours[:0x7F]
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0 and pos[1] == 2.0 ** -9


def wide_range_blocks(rng, rows, cols):
    """Blocks whose magnitudes span many binades, with zero blocks, exact
    powers of two as amax, and elements that saturate."""
    a = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-20, 20, (rows, 1)))
    a *= np.exp2(rng.integers(-12, 1, (rows, cols)))            # spread inside a block
    a = a.astype(np.float32)
    a[0, :32] = 0.0                                               # all-zero block
    a[1, :32] = 0.0
    a[1, 5] = 4.0                                                 # amax exactly a power of two
    a[1, 6] = -3.999                                              # just below it: 3.999 / 2^-6 = 255.9
    a[2, :32] = 1.0
    a[2, 3] = 1.99                                                # 1.99 / 2^-8 = 509 -> saturates to 448
    a[3, 32:64] = -1e-3                                           # negative block
    a[3, 40] = -1e-30                                             # rounds to zero with sign kept
    return a


def expected_scales(a):
    """E8M0 byte per 32-block from numpy's frexp: floor(log2 amax) - 8."""
    blocks = np.abs(a.astype(np.float64)).reshape(a.shape[0], -1, 32).max(-1)
    _, e = np.frexp(blocks)
    s = np.clip(e - 1 - 8, -127, 127)
    s = np.where(blocks == 0, -127, s)
    return (s + 127).astype(np.uint8)


@pytest.mark.parametrize("src", ["f32", "bf16"])
def test_quantize_matches_frexp_and_torch(src):
    rng = np.random.default_rng(7)
    a = wide_range_blocks(rng, 64, 256)
    if src == "bf16":
        a_in = (torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
        a = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    else:
        a_in = a
    codes, scales = oracle.mxfp8_quantize(a_in)
    assert np.array_equal(scales, expected_scales(a))
    X = np.ldexp(1.0, np.repeat(scales.astype(np.int64), 32, axis=1) - 127)
    scaled = (a.astype(np.float64) / X).astype(np.float32)  # exact: power-of-two scaling
    assert np.array_equal(codes, torch_e4m3_encode(scaled))
    # the scale property: amax / X in [256, 512) for every non-zero block
    amax = np.abs(a.astype(np.float64)).reshape(64, -1, 32).max(-1)
    r = amax / np.ldexp(1.0, scales.astype(np.int64) - 127)
    nz = amax > 0
    assert np.all((r[nz] >= 256) & (r[nz] < 512))
    assert np.all(scales[~nz] == 0)
    assert codes[0, :32].tolist() == [0] * 32
    assert codes[2, 3] == 0x7E                                      # saturated
    assert codes[3, 40] == 0x80                                     # -0 keeps its sign


def test_quantize_is_nearest_code_brute_force():
    rng = np.random.default_rng(3)
    a = wide_range_blocks(rng, 8, 64)
    codes, scales = oracle.mxfp8_quantize(a)
    X = np.ldexp(1.0, np.repeat(scales.astype(np.int64), 32, axis=1) - 127)
    q = a.astype(np.float64) / X
    vals = oracle.e4m3_value(np.arange(256))
    finite = np.arange(256)[~np.isnan(vals)]
    for (i, j), v in np.ndenumerate(q):
        dist = np.abs(vals[finite] - min(max(v, -448.0), 448.0))
        best = finite[dist == dist.min()]
        best_vals = set(vals[best].tolist())
        got = int(codes[i, j])
        assert vals[got] in best_vals, (i, j, v)
        if len(best_vals) > 1:  # a tie between two values: the even mantissa wins
            assert got & 1 == 0, (i, j, v)


def test_quantize_error_bound():
    rng = np.random.default_rng(11)
    a = wide_range_blocks(rng, 128, 128)
    codes, scales = oracle.mxfp8_quantize(a)
    X = np.ldexp(1.0, np.repeat(scales.astype(np.int64), 32, axis=1) - 127)
    d = oracle.mxfp8_decode(codes, scales)
    v = a.astype(np.float64)
    err = np.abs(d - v)
    normal = np.abs(v) >= X * 2.0 ** -6
    sat = np.abs(v) >= X * 448
    assert np.all(err[normal & ~sat] <= np.abs(v[normal & ~sat]) * 2.0 ** -4)
    assert np.all(err[~normal] <= X[~normal] * 2.0 ** -10)
    assert np.all(err[sat] <= X[sat] * 64)


def test_quantize_exact_round_trip():
    """Blocks built from codes and a scale, with the largest magnitude in
    [256, 448], come back as the same codes and scale."""
    rng = np.random.default_rng(5)
    vals = oracle.e4m3_value(np.arange(256))
    finite = np.arange(256)[~np.isnan(vals)]
    big = [c for c in range(0x7F) if 256 <= vals[c] <= 448]
    rows, nb = 16, 4
    codes = rng.choice(finite, size=(rows, nb * 32)).astype(np.uint8)
    for r in range(rows):
        for b in range(nb):
            blk = codes[r, b * 32:(b + 1) * 32]
            blk[np.abs(vals[blk]) > 448] = 0
            blk[rng.integers(0, 32)] = rng.choice(big) | (0x80 if rng.random() < 0.5 else 0)
            codes[r, b * 32:(b + 1) * 32] = blk
    scales = rng.integers(127 - 20, 127 + 20, (rows, nb)).astype(np.uint8)
    a = oracle.mxfp8_decode(codes, scales).astype(np.float32)
    c2, s2 = oracle.mxfp8_quantize(a)
    assert np.array_equal(s2, scales)
    # a zero value may come back as -0 (0x80) only if it was -0; compare values and codes
    assert np.array_equal(c2, codes)


def silu(z):
    return z / (1.0 + np.exp(-z))


def numpy_mx(a32):
    """Independent MXFP8 quantise-and-decode: frexp scale, torch rounding."""
    s = expected_scales(a32)
    X = np.ldexp(1.0, np.repeat(s.astype(np.int64), 32, axis=-1) - 127)
    c = torch_e4m3_encode((a32.astype(np.float64) / X).astype(np.float32))
    return torch_e4m3_decode(c) * X


def test_ffn_mxfp8_matches_float64_numpy():
    rng = np.random.default_rng(13)
    E, H, I, R = 3, 64, 96, 20
    x = rng.standard_normal((R, H)).astype(np.float32)
    wg = (rng.standard_normal((E, I, H)) / np.sqrt(H)).astype(np.float32)
    wu = (rng.standard_normal((E, I, H)) / np.sqrt(H)).astype(np.float32)
    wd = (rng.standard_normal((E, H, I)) / np.sqrt(I)).astype(np.float32)
    offsets = np.array([0, 7, 7, R], np.int32)  # expert 1 gets no rows
    xq = oracle.mxfp8_quantize(x)
    W = {n: oracle.mxfp8_quantize(w) for n, w in (("gate", wg), ("up", wu), ("down", wd))}
    y = oracle.grouped_ffn_mxfp8(*xq, offsets, W["gate"], W["up"], W["down"])
    xd = oracle.mxfp8_decode(*xq)
    Wd = {n: oracle.mxfp8_decode(*W[n]) for n in W}
    ref = np.zeros((R, H))
    for e in range(E):
        rows = slice(offsets[e], offsets[e + 1])
        if offsets[e] == offsets[e + 1]:
            continue
        a = xd[rows] @ Wd["gate"][e].T
        u = xd[rows] @ Wd["up"][e].T
        h = numpy_mx((silu(a) * u).astype(np.float32))
        ref[rows] = h @ Wd["down"][e].T
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(y - ref)) <= 1e-5 * rms
    # the subset interface returns the same rows
    sub = oracle.grouped_ffn_mxfp8(*xq, offsets, W["gate"], W["up"], W["down"], rows=np.array([19, 0, 8]))
    assert np.array_equal(sub, y[[19, 0, 8]])
    # and the 8-bit FFN stays near the unquantised one (a wrong scale sign or
    # block index would not)
    y32 = oracle.grouped_ffn(x, offsets, wg, wu, wd)
    assert np.sqrt(np.mean((y - y32) ** 2)) <= 0.1 * np.sqrt(np.mean(y32 ** 2))


def test_layer_mxfp8_routing_is_the_high_precision_routing():
    import workloads as W
    cfg = W.CONFIGS["qwen3_skewed"].with_tokens(64).replace(hidden=128, inter=64, experts=16)
    inp = {k: W.to_numpy_raw(v) for k, v in W.make_layer_inputs(cfg, "cpu").items()}
    wq = {n: oracle.mxfp8_quantize(inp[f"w_{n}"]) for n in ("gate", "up", "down")}
    kw = dict(bias=inp["bias"], k_per_token=inp["k_per_token"], capacity_factor=cfg.capacity_factor)
    got = oracle.layer_forward_mxfp8(inp["x"], inp["w_router"], wq, cfg.top_k, **kw)
    ref = oracle.layer_forward(inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"],
                               cfg.top_k, **kw)
    for key in ("ids", "row_of_slot", "offsets"):
        assert np.array_equal(got[key], ref[key])
    assert np.array_equal(got["gates"], ref["gates"])
    err = np.sqrt(np.mean((got["out"] - ref["out"]) ** 2))
    assert err <= 0.1 * np.sqrt(np.mean(ref["out"] ** 2))
    # tokens subset
    sub = oracle.layer_forward_mxfp8(inp["x"], inp["w_router"], wq, cfg.top_k, tokens=[63, 2], **kw)
    assert np.array_equal(sub["out"], got["out"][[63, 2]])


@pytest.mark.parametrize("tokens", [None, [17, 0, 5]])
def test_layer_mxfp8_with_shared_expert_matches_float64_numpy(tokens):
    """The MXFP8 layer with a shared expert, composed independently in
    float64 numpy: each token's x quantised on its own (frexp scales, torch
    E4M3 rounding), every kept slot's expert FFN on the decoded codes with h
    re-quantised along I, the gate-weighted sum over the slots in order, and
    the shared expert's FFN on the same quantised x added last with weight 1
    (not scaled by the routed scale).  Routing (ids, gates, kept slots) is the
    high-precision routing pinned elsewhere; dropping the shared term, scaling
    it by 2.5, or quantising the shared expert's x with other scales fails."""
    import workloads as W
    cfg = W.CONFIGS["deepseek_v3"].with_tokens(24).replace(hidden=128, inter=64, experts=16, top_k=4,
                                                           num_groups=4, topk_groups=2, shared_inter=96)
    inp = {k: W.to_numpy_raw(v) for k, v in W.make_layer_inputs(cfg, "cpu", salt=4).items()}
    wq = {n: oracle.mxfp8_quantize(inp[f"w_{n}"]) for n in ("gate", "up", "down")}
    sq = {n: oracle.mxfp8_quantize(inp[f"ws_{n}"]) for n in ("gate", "up", "down")}
    got = oracle.layer_forward_mxfp8(inp["x"], inp["w_router"], wq, cfg.top_k, bias=inp["bias"],
                                     score=cfg.score, routed_scale=cfg.routed_scale, num_groups=cfg.num_groups,
                                     topk_groups=cfg.topk_groups, group_topn=cfg.group_topn, shared=sq,
                                     tokens=tokens)
    x32 = W.bf16_bits_to_f32(inp["x"])
    dec = {n: torch_e4m3_decode(wq[n][0]) * np.ldexp(1.0, np.repeat(wq[n][1].astype(np.int64), 32, -1) - 127)
           for n in wq}
    sdec = {n: torch_e4m3_decode(sq[n][0]) * np.ldexp(1.0, np.repeat(sq[n][1].astype(np.int64), 32, -1) - 127)
            for n in sq}

    def ffn(xd, g, u, d):
        h = numpy_mx((silu(xd @ g.T) * (xd @ u.T)).astype(np.float32))
        return h @ d.T

    toks = range(cfg.tokens) if tokens is None else tokens
    ref = np.zeros((len(toks), cfg.hidden))
    shared_part = np.zeros_like(ref)
    for q, t in enumerate(toks):
        xd = numpy_mx(x32[t][None])           # this token's x alone: per-token scales
        for j in range(cfg.top_k):
            if got["row_of_slot"][t, j] < 0:
                continue
            e = got["ids"][t, j]
            ref[q] += float(got["gates"][t, j]) * ffn(xd, dec["gate"][e], dec["up"][e], dec["down"][e])[0]
        shared_part[q] = ffn(xd, sdec["gate"], sdec["up"], sdec["down"])[0]
    full = ref + shared_part
    r = np.sqrt(np.mean(full ** 2))
    assert np.max(np.abs(got["out"] - full)) <= 1e-5 * r
    # the shared term is a sizeable part of the output (so a dropped or
    # mis-scaled term cannot hide inside the tolerance)
    assert np.sqrt(np.mean(shared_part ** 2)) >= 0.2 * r
    assert np.max(np.abs(got["out"] - (ref + 2.5 * shared_part))) > 1e-2 * r
    assert np.isclose(got["gates"].sum(1), cfg.routed_scale, rtol=1e-6).all()
