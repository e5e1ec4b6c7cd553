"""The expert-parallel exchange over G virtual ranks on one GPU, through the C
ABI, against the CPU oracle.

* moe_ep_dispatch_layout: rank counts and offsets, the token of every send
  row, the local expert ids and gates each row carries, and every slot's
  send row, bit-exact against the oracle's layout on the same ids and gates
  (rows past the rows sent cleared); the payload rows bit-identical to the
  tokens' x rows.
* The exchange chain: layout, then on every virtual rank the step chain
  moe_dispatch / moe_grouped_ffn / moe_combine over the rows it received,
  with its local expert ids and only its own experts' weights (one
  pre-reduced row per received row), then moe_ep_combine at the source.
  Its output must match the oracle layer routed on the same logits within
  2e-2 * RMS, and moe_layer_forward's within 5e-3 * RMS (the same FFN rows,
  cut into other row tiles).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from expert_serving_amd import abi

from gpu_util import assert_close_rms, dev, host, i32, rms, say, workspace
from test_gpu_layer import check_routing, gpu_layer, oracle_inputs
from test_oracle_ep import random_routing

pytestmark = pytest.mark.gpu


def gpu_layout(shape, G, ids_d, gates_d, x=None):
    T, k = shape.num_tokens, shape.top_k
    n_rows = T * min(k, G)
    ws = workspace(shape)
    out = dict(rank_counts=i32(G, -7), rank_offsets=i32(G + 1, -7), send_token=i32(max(n_rows, 1), -7),
               send_ids=i32(max(n_rows * k, 1), -7),
               send_gates=torch.full((max(n_rows * k, 1),), 7.0, dtype=torch.float32, device=dev()),
               slot_send_pos=i32(max(T * k, 1), -7))
    send_x = None if x is None else torch.empty(max(n_rows, 1), shape.hidden, dtype=x.dtype, device=dev())
    abi.moe_ep_dispatch_layout(shape, G, ids_d, gates_d, x, out["rank_counts"], out["rank_offsets"],
                               out["send_token"], out["send_ids"], out["send_gates"], out["slot_send_pos"], send_x,
                               ws)
    flags = abi.moe_read_device_flags(ws)
    res = {key: v.cpu().numpy() for key, v in out.items()}
    res["send_token"] = res["send_token"][:n_rows]
    res["send_ids"] = res["send_ids"][:n_rows * k].reshape(n_rows, k)
    res["send_gates"] = res["send_gates"][:n_rows * k].reshape(n_rows, k)
    res["slot_send_pos"] = res["slot_send_pos"][:T * k].reshape(T, k)
    res["flags"] = flags
    return res, send_x


def check_layout(got, ids, gates, E, G, what):
    ref = oracle.ep_layout(ids, gates, E, G)
    for key in ("rank_counts", "rank_offsets", "send_token", "send_ids", "slot_send_pos"):
        assert np.array_equal(got[key], ref[key]), f"{what}: {key} differs"
    assert np.array_equal(got["send_gates"].view(np.uint32), ref["send_gates"].view(np.uint32)), what
    return ref


LAYOUT_CASES = [
    # T, E, k, G
    (1, 8, 2, 2), (63, 8, 2, 4), (65, 16, 4, 4), (1000, 8, 2, 8), (4096, 8, 2, 2),
    (2049, 256, 8, 8), (777, 64, 6, 64), (300, 32, 8, 1), (513, 128, 8, 16), (4096, 16, 16, 16),
]


@pytest.mark.parametrize("T,E,k,G", LAYOUT_CASES, ids=[f"T{c[0]}-E{c[1]}-k{c[2]}-G{c[3]}" for c in LAYOUT_CASES])
def test_ep_layout_bit_exact(T, E, k, G):
    say(f"ep layout T={T} E={E} k={k} G={G}")
    ids, gates = random_routing(T, E, k, seed=T * 7 + G)
    shape = abi.make_shape(num_tokens=T, hidden=64, num_experts=E, intermediate=64, top_k=k)
    got, _ = gpu_layout(shape, G, torch.from_numpy(ids).to(dev()), torch.from_numpy(gates).to(dev()))
    assert got["flags"] == 0
    ref = check_layout(got, ids, gates, E, G, f"T={T} E={E} k={k} G={G}")
    say(f"  rows sent {ref['S']} of {int((ids >= 0).sum())} routed slots; per rank {ref['rank_counts'].tolist()[:8]}")


def test_ep_layout_flags_invalid_ids():
    T, E, k, G = 300, 16, 4, 4
    ids, gates = random_routing(T, E, k, seed=5)
    ids[7, 0] = E + 3
    ids[100, 2] = -5
    shape = abi.make_shape(num_tokens=T, hidden=64, num_experts=E, intermediate=64, top_k=k)
    got, _ = gpu_layout(shape, G, torch.from_numpy(ids).to(dev()), torch.from_numpy(gates).to(dev()))
    assert got["flags"] & abi.MOE_FLAG_BAD_EXPERT
    clean = np.where((ids >= 0) & (ids < E), ids, -1).astype(np.int32)
    check_layout(got, clean, gates, E, G, "invalid ids")
    assert got["slot_send_pos"][7, 0] == -1 and got["slot_send_pos"][100, 2] == -1


def test_ep_layout_of_deepseek_v3_routing_and_payload():
    """The DeepSeek-V3-shaped workload's own routing (8192 tokens, group-limited
    to 4 of 8 groups) over the EP=8 layout: a token reaches at most 4 ranks;
    the payload rows are the tokens' x rows, bit for bit."""
    cfg = W.CONFIGS["deepseek_v3"]
    inp = W.make_layer_inputs(cfg, dev())
    g = gpu_layer(cfg, inp)
    G = 8
    shape = abi.make_shape(cfg)
    ids_d = torch.from_numpy(g["ids"]).to(dev())
    gates_d = torch.from_numpy(g["gates"]).to(dev())
    got, send_x = gpu_layout(shape, G, ids_d, gates_d, inp["x"])
    assert got["flags"] == 0
    ref = check_layout(got, g["ids"], g["gates"], cfg.experts, G, "deepseek_v3")
    S = ref["S"]
    per_token = np.bincount(got["send_token"][:S], minlength=cfg.tokens)
    assert per_token.max() <= cfg.topk_groups
    idx = torch.from_numpy(got["send_token"][:S].astype(np.int64)).to(dev())
    assert torch.equal(send_x[:S], inp["x"][idx])
    routed = int((g["ids"] >= 0).sum())
    say(f"  rows sent {S} (per rank {ref['rank_counts'].tolist()}) for {routed} routed slots: "
        f"{S / routed:.3f} of the per-expert copies")


def run_chain(cfg, inp, g, G):
    """The exchange over G virtual ranks with the library's entry points; the
    ranks' counts are read back to size their step calls (whose shapes have
    E/G experts, so top_k <= E/G)."""
    T, E, k, H = cfg.tokens, cfg.experts, cfg.top_k, cfg.hidden
    epr = E // G
    shape = abi.make_shape(cfg)
    ids_d = torch.from_numpy(g["ids"]).to(dev())
    gates_d = torch.from_numpy(g["gates"]).to(dev())
    lay, send_x = gpu_layout(shape, G, ids_d, gates_d, inp["x"])
    n_rows = T * min(k, G)
    send_ids = torch.from_numpy(lay["send_ids"]).to(dev())
    send_gates = torch.from_numpy(lay["send_gates"]).to(dev())
    partial = torch.zeros(max(n_rows, 1), H, dtype=torch.float32, device=dev())
    for d in range(G):
        a, b = int(lay["rank_offsets"][d]), int(lay["rank_offsets"][d + 1])
        n = b - a
        if n == 0:
            continue
        sd = abi.make_shape(num_tokens=n, hidden=H, num_experts=epr, intermediate=cfg.inter, top_k=k,
                            act_dtype=cfg.dtype)
        wsd = workspace(sd)
        counts, offsets, ros, rt = i32(epr), i32(epr + 1), i32(n * k), i32(n * k)
        x_perm = torch.empty(n * k, H, dtype=inp["x"].dtype, device=dev())
        abi.moe_dispatch(sd, send_x[a:b], send_ids[a:b], counts, offsets, ros, rt, None, x_perm, wsd)
        y = torch.empty(n * k, H, dtype=torch.float32, device=dev())
        sl = slice(d * epr, (d + 1) * epr)
        abi.moe_grouped_ffn(sd, x_perm, offsets, inp["w_gate"][sl], inp["w_up"][sl], inp["w_down"][sl], y, wsd)
        abi.moe_combine(sd, y, ros, send_gates[a:b], None, partial[a:b])
    y_sh = None
    if cfg.shared_inter:
        ss = abi.make_shape(num_tokens=T, hidden=H, num_experts=1, intermediate=cfg.shared_inter, top_k=1,
                            act_dtype=cfg.dtype)
        y_sh = torch.empty(T, H, dtype=torch.float32, device=dev())
        abi.moe_grouped_ffn(ss, inp["x"], torch.tensor([0, T], dtype=torch.int32, device=dev()), inp["ws_gate"][None],
                            inp["ws_up"][None], inp["ws_down"][None], y_sh, workspace(ss))
    out = torch.empty(T, H, dtype=torch.float32, device=dev())
    abi.moe_ep_combine(shape, G, partial, torch.from_numpy(lay["slot_send_pos"]).to(dev()), y_sh, out)
    torch.cuda.synchronize()
    return out, lay


CHAIN_CASES = [("deepseek_v3", 512, 8), ("deepseek_v3", 2048, 2), ("mixtral_prefill", 256, 4),
               ("mixtral_decode", 64, 4), ("qwen3_skewed", 1024, 8)]


@pytest.mark.parametrize("name,T,G", CHAIN_CASES, ids=[f"{c[0]}-T{c[1]}-G{c[2]}" for c in CHAIN_CASES])
def test_ep_exchange_chain_matches_the_layer(name, T, G):
    cfg = W.CONFIGS[name].with_tokens(T)
    if cfg.capacity_factor > 0:
        cfg = cfg.replace(capacity_factor=0.0)   # capacity is the receiving rank's; compared without it
    say(f"ep chain {name} T={T} G={G}")
    inp = W.make_layer_inputs(cfg, dev(), salt=13)
    g = gpu_layer(cfg, inp)
    check_routing(cfg, g, inp)
    out, lay = run_chain(cfg, inp, g, G)
    full = g["out"].cpu().numpy()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    assert_close_rms(got, full, 5e-3, f"{name} exchange chain vs moe_layer_forward")
    tokens = np.arange(T, dtype=np.int32)
    oi = oracle_inputs(cfg, inp, tokens, g["ids"])
    ref = oracle.layer_forward_cfg(cfg, oi, tokens=tokens, logits=g["logits"])
    assert_close_rms(got, ref["out"], 2e-2, f"{name} exchange chain vs oracle")
    routed = int((g["ids"] >= 0).sum())
    say(f"  rows sent {int(lay['rank_offsets'][-1])} for {routed} routed slots over {G} ranks")
