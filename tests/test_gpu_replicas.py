"""Redundant experts on the GPU: moe_map_replicas against the oracle
(bit-exact), and the invariant that sending slots to identical replicas
leaves the layer output unchanged -- the step-API chain route -> replica map
-> dispatch -> grouped FFN -> combine over the physical experts reproduces
moe_layer_forward on the logical experts bit for bit (every row's arithmetic
is the same; only the row grouping changes; where the layer keeps its expert
outputs in fp16, the chain's y is rounded the same way before its combine)."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from expert_serving_amd import abi

from gpu_util import dev, f32, host, i32, say, workspace

pytestmark = pytest.mark.gpu


def hot_table(counts, n_hot, extra, seed):
    """Replica table giving the n_hot most loaded experts `extra` more copies,
    physical ids shuffled so replicas are not adjacent."""
    E = len(counts)
    hot = np.argsort(-counts, kind="stable")[:n_hot]
    n = np.ones(E, np.int64)
    n[hot] += extra
    off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    P = int(off[-1])
    rex = np.random.default_rng(seed).permutation(P).astype(np.int32)
    return off, rex, P


def gpu_map(shape, ids, off, rex, P):
    ws = workspace(shape)
    ids_t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(dev())
    phys = i32(ids.size, -9)
    abi.moe_map_replicas(shape, ids_t, torch.from_numpy(off).to(dev()), torch.from_numpy(rex).to(dev()), P,
                         phys, ws)
    return phys.cpu().numpy().reshape(ids.shape), abi.moe_read_device_flags(ws)


MAP_CASES = [
    # name, T, E, k, k choices, zipf, hot experts, extra copies
    ("deepseek_shaped", 8192, 256, 8, None, 1.1, 16, 2),
    ("qwen_per_token_k", 4096, 128, 8, (2, 4, 6, 8), 1.2, 8, 3),
    ("single_tile", 100, 8, 2, None, 0.8, 2, 1),
    ("identity", 2000, 16, 4, None, 0.0, 0, 0),
]


@pytest.mark.parametrize("name,T,E,k,kch,zipf,n_hot,extra", MAP_CASES, ids=[c[0] for c in MAP_CASES])
def test_map_replicas_matches_oracle(name, T, E, k, kch, zipf, n_hot, extra):
    bias = W.log_zipf_bias(E, zipf) if zipf > 0 else None
    logits = W.make_logits(T, E, seed=17, bias=bias).numpy()
    kpt = W.make_k_per_token(T, kch, seed=3).numpy() if kch else None
    ids, _ = oracle.route(logits, k, kpt)
    counts = np.bincount(ids[ids >= 0], minlength=E)
    off, rex, P = hot_table(counts, n_hot, extra, seed=5)
    if name == "identity":
        rex = np.arange(P, dtype=np.int32)
    say(f"replica map {name}: T={T} E={E} k={k} physical={P}")
    shape = abi.make_shape(num_tokens=T, hidden=64, num_experts=E, intermediate=64, top_k=k)
    got, flags = gpu_map(shape, ids, off, rex, P)
    ref, bad = oracle.map_replicas(ids, off, rex, P)
    assert bad == 0 and flags == 0
    assert np.array_equal(got, ref)
    if name == "identity":
        assert np.array_equal(got, np.where(ids >= 0, ids, -1))
    pc = np.bincount(got[got >= 0], minlength=P)
    say(f"  max/mean load: logical {counts.max() / counts.mean():.2f} -> physical {pc.max() / pc.mean():.2f}")


def test_map_replicas_invalid_table_flagged():
    T, E, k = 300, 6, 2
    ids, _ = oracle.route(W.make_logits(T, E, seed=8).numpy(), k)
    off = np.array([0, 1, 1, 3, 4, 5, 6], np.int32)      # expert 1: no replica
    rex = np.array([0, 1, 9, 2, 3, 4], np.int32)         # expert 2's second replica: out of range
    shape = abi.make_shape(num_tokens=T, hidden=64, num_experts=E, intermediate=64, top_k=k)
    got, flags = gpu_map(shape, ids, off, rex, 5)
    ref, bad = oracle.map_replicas(ids, off, rex, 5)
    assert bad > 0 and flags == abi.MOE_FLAG_BAD_REPLICA
    assert np.array_equal(got, ref)


def replicated(w, logical_of_phys):
    return torch.index_select(w, 0, torch.from_numpy(logical_of_phys).long().to(w.device)).contiguous()


@pytest.mark.parametrize("name,T", [("qwen3_skewed", 512), ("deepseek_v3", 256)])
def test_replicated_chain_reproduces_layer(name, T):
    # no capacity: a capacity per physical expert would drop differently
    cfg = W.CONFIGS[name].replace(capacity_factor=0.0).with_tokens(T)
    say(f"replicated chain {name} T={T}")
    inp = W.make_layer_inputs(cfg, dev(), salt=7)
    E, k, H = cfg.experts, cfg.top_k, cfg.hidden
    shape = abi.make_shape(cfg)
    ws = workspace(shape)
    ref = torch.empty(T, H, dtype=torch.float32, device=dev())
    ids = i32(T * k)
    gates = f32(T * k)
    abi.moe_layer_forward(shape, inp["x"], inp["w_router"], inp["bias"], inp["k_per_token"], inp["w_gate"],
                          inp["w_up"], inp["w_down"], inp["ws_gate"], inp["ws_up"], inp["ws_down"], ref,
                          dict(topk_ids=ids, topk_gates=gates), ws)
    counts = np.bincount(host(ids)[host(ids) >= 0], minlength=E)
    off, rex, P = hot_table(counts, 8, 2, seed=1)
    logical_of_phys = np.empty(P, np.int64)
    for e in range(E):
        logical_of_phys[rex[off[e]:off[e + 1]]] = e
    # the chain over physical experts
    phys = i32(T * k)
    abi.moe_map_replicas(shape, ids, torch.from_numpy(off).to(dev()), torch.from_numpy(rex).to(dev()), P, phys, ws)
    assert abi.moe_read_device_flags(ws) == 0
    sp = abi.make_shape(cfg, num_experts=P, num_groups=1, topk_groups=1, group_topn=0)
    wsp = workspace(sp)
    counts_p, offsets_p = i32(P), i32(P + 1)
    ros, row_token, nd = i32(T * k), i32(T * k), i32(1)
    x_perm = torch.empty(T * k, H, dtype=inp["x"].dtype, device=dev())
    abi.moe_dispatch(sp, inp["x"], phys, counts_p, offsets_p, ros, row_token, nd, x_perm, wsp)
    y = torch.empty(T * k, H, dtype=torch.float32, device=dev())
    abi.moe_grouped_ffn(sp, x_perm, offsets_p, replicated(inp["w_gate"], logical_of_phys),
                        replicated(inp["w_up"], logical_of_phys), replicated(inp["w_down"], logical_of_phys), y, wsp)
    y_shared = None
    if cfg.shared_inter > 0:
        # the shared expert through the step API: one expert over all T rows of x
        s1 = abi.make_shape(num_tokens=T, hidden=H, num_experts=1, intermediate=cfg.shared_inter, top_k=1,
                            act_dtype=shape.act_dtype)
        ws1 = workspace(s1)
        y_shared = torch.empty(T, H, dtype=torch.float32, device=dev())
        abi.moe_grouped_ffn(s1, inp["x"], torch.tensor([0, T], dtype=torch.int32, device=dev()),
                            inp["ws_gate"].unsqueeze(0).contiguous(), inp["ws_up"].unsqueeze(0).contiguous(),
                            inp["ws_down"].unsqueeze(0).contiguous(), y_shared, ws1)
    out = torch.empty(T, H, dtype=torch.float32, device=dev())
    abi.moe_combine(sp, y, ros, gates, y_shared, out, None)
    # the layer keeps the expert outputs in fp16 when its down projection is
    # not split: the same chain with y (and the shared y) rounded to fp16
    out16 = torch.empty(T, H, dtype=torch.float32, device=dev())
    abi.moe_combine(sp, y.half().float(), ros, gates, None if y_shared is None else y_shared.half().float(),
                    out16, None)
    torch.cuda.synchronize()
    pc = np.bincount(host(phys)[host(phys) >= 0], minlength=P)
    say(f"  physical experts {P}; max/mean load {counts.max() / counts.mean():.2f} -> {pc.max() / pc.mean():.2f}")
    same32, same16 = torch.equal(out, ref), torch.equal(out16, ref)
    say(f"  layer equals the chain with fp32 y: {same32}, with fp16 y: {same16}")
    assert same32 or same16, f"max |diff| {float((out - ref).abs().max())} / {float((out16 - ref).abs().max())}"
