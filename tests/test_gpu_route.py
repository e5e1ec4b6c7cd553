"""GPU parity of routing (S1 router logits, S2 scoring/top-k/gates) and of the
group-score sigmoid, through the C ABI, against the CPU oracle.

Routing is compared bit-exactly given the same fp32 logits (ties to the lower
expert index); gates within 1e-6 relative.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from expert_serving_amd import abi

from gpu_util import assert_close_rms, dev, f32, host, i32, say, workspace

pytestmark = pytest.mark.gpu


def test_group_score_sigmoid_bitwise():
    # every 7th fp32 bit pattern in [0, 30] and its negation, plus edges
    pos = np.arange(0, 0x41F00001, 7, dtype=np.uint32)
    extra = np.array([0x41F00000, 0x41F00001, 0x42C80000, 0x7F7FFFFF, 0x00000001, 0x3F800000], np.uint32)
    bits = np.concatenate([pos, extra])
    x = np.concatenate([bits.view(np.float32), -bits.view(np.float32)])
    say(f"  sigmoid: {x.size} values")
    ref = oracle.sigmoid_spec(x)
    chunk = 1 << 26
    for i in range(0, x.size, chunk):
        xd = torch.from_numpy(x[i:i + chunk]).to(dev())
        yd = torch.empty_like(xd)
        abi.moe_group_score_sigmoid(xd, yd)
        got = yd.cpu().numpy()
        bad = np.nonzero(got.view(np.uint32) != ref[i:i + chunk].view(np.uint32))[0]
        assert bad.size == 0, f"{bad.size} mismatches, first x={x[i + bad[0]]!r}"


ROUTE_CASES = [
    # name, T, E, k, options
    ("softmax_e8_k2_ties", 1001, 8, 2, dict(tie=0.3)),
    ("softmax_e5_k1_ties", 513, 5, 1, dict(tie=0.5)),
    ("softmax_e64_k16", 300, 64, 16, dict(tie=0.1)),
    ("softmax_e512_k16_norenorm", 200, 512, 16, dict(renorm=0)),
    ("softmax_e512_k3", 129, 512, 3, dict(tie=0.2)),
    ("single_token", 1, 8, 2, dict()),
    ("deepseek_full_T", 8192, 256, 8, dict(score=1, scale=2.5, G=8, keep=4, topn=2, zipf=1.1)),
    ("deepseek_topn1", 2000, 256, 8, dict(score=1, scale=2.5, G=8, keep=4, topn=1, zipf=1.1, tie=0.05)),
    ("grouped_e96_g3", 777, 96, 6, dict(score=1, G=3, keep=2, topn=2, tie=0.1)),
    ("grouped_softmax_e64_g8", 500, 64, 4, dict(G=8, keep=3, topn=2)),
    # groups on 16 lanes, top-4 group scores (butterfly merge of 4-long lists)
    ("grouped_e128_g4_topn4", 600, 128, 8, dict(score=1, G=4, keep=2, topn=4, tie=0.1)),
    # 12 experts per group (not a power-of-two run of lanes): groups scored serially
    ("grouped_e48_g4_serial", 300, 48, 4, dict(score=1, G=4, keep=2, topn=3, tie=0.1)),
    ("sigmoid_norenorm", 400, 32, 4, dict(score=1, renorm=0)),
    ("qwen_per_token_k", 16384, 128, 8, dict(kpt=(2, 4, 6, 8), zipf=1.2)),
    ("per_token_k_invalid", 999, 16, 8, dict(kpt=(1, 3, 8), bad_k=True)),
]


@pytest.mark.parametrize("name,T,E,k,o", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_parity_given_logits(name, T, E, k, o):
    say(f"route case {name}: T={T} E={E} k={k} {o}")
    bias = W.log_zipf_bias(E, o["zipf"]) if "zipf" in o else None
    logits = W.make_logits(T, E, seed=zlib.crc32(name.encode()) & 0xFFFF, bias=bias, tie_fraction=o.get("tie", 0.0))
    kpt = None
    if "kpt" in o:
        kpt = W.make_k_per_token(T, o["kpt"], seed=7)
        if o.get("bad_k"):
            kpt[::97] = 0
            kpt[3::101] = k + 1
    score, renorm, scale = o.get("score", 0), o.get("renorm", 1), o.get("scale", 1.0)
    G, keep, topn = o.get("G", 1), o.get("keep", 1), o.get("topn", 0)
    ids_o, gates_o = oracle.route(logits.numpy(), k, None if kpt is None else kpt.numpy(), score, renorm,
                                  scale, G, keep, topn)
    shape = abi.make_shape(num_tokens=T, hidden=64, num_experts=E, intermediate=64, top_k=k, score=score,
                           renormalize=renorm, routed_scale=scale, num_groups=G, topk_groups=keep,
                           group_topn=topn)
    ws = workspace(shape)
    ids = i32(T * k, -7)
    gates = f32(T * k)
    ld = logits.to(dev())
    abi.moe_route_topk(shape, None, None, None, ld, None, None if kpt is None else kpt.to(dev()), ids, gates, ws)
    flags = abi.moe_read_device_flags(ws)
    ids_g = ids.cpu().numpy().reshape(T, k)
    gates_g = gates.cpu().numpy().reshape(T, k)
    mism = np.nonzero((ids_g != ids_o).any(1))[0]
    assert mism.size == 0, f"{mism.size} tokens differ; first t={mism[0]}: gpu {ids_g[mism[0]]} oracle {ids_o[mism[0]]}"
    np.testing.assert_allclose(gates_g, gates_o, rtol=1e-6, atol=1e-30)
    assert flags == (abi.MOE_FLAG_BAD_K if o.get("bad_k") else 0)


# (dtype, T, H, E, bias): bf16 layers with E <= 32 take the vector-ALU router
# (one token per block below 1024 tokens, several above), the rest the MFMA
# GEMM; ragged token counts, one-chunk rows (H = 64) and E below the
# kernel's expert bound are all covered
ROUTER_CASES = [
    (W.DT_BF16, 1000, 4096, 8, True),
    (W.DT_BF16, 1024, 4096, 8, True),
    (W.DT_BF16, 4099, 4096, 8, False),
    (W.DT_BF16, 1, 4096, 8, True),
    (W.DT_BF16, 130, 2048, 5, True),
    (W.DT_BF16, 1027, 2048, 16, True),
    (W.DT_BF16, 70, 1024, 13, False),
    (W.DT_BF16, 2050, 1024, 32, True),
    (W.DT_BF16, 3, 64, 24, True),
    (W.DT_BF16, 257, 2048, 33, True),
    # E > 32 with at most 1024 tokens: vector-ALU router over 8-expert
    # slices (one token per block below 64 tokens, four from 64)
    (W.DT_BF16, 1, 7168, 256, True),
    (W.DT_BF16, 63, 2048, 128, False),
    (W.DT_BF16, 256, 7168, 256, True),
    (W.DT_BF16, 100, 1024, 37, True),
    (W.DT_BF16, 5, 512, 512, True),
    (W.DT_BF16, 777, 7168, 256, True),
    (W.DT_BF16, 4096, 2048, 128, True),
    (W.DT_BF16, 16384, 1024, 256, True),      # 128-row tiles (8-wave MFMA kernel)
    (W.DT_BF16, 8192, 1024, 64, True),        # the smallest token count on 128-row tiles
    (W.DT_F32, 300, 512, 8, True),
]


@pytest.mark.parametrize("dt,T,H,E,with_bias", ROUTER_CASES,
                         ids=[f"{'bf16' if c[0] == W.DT_BF16 else 'f32'}-T{c[1]}-H{c[2]}-E{c[3]}" for c in ROUTER_CASES])
def test_router_logits_parity(dt, T, H, E, with_bias):
    say(f"router logits dtype={dt} T={T} H={H} E={E} bias={with_bias}")
    x = W.normal((T, H), 1.0, dt, dev(), 11)
    wr = W.normal((E, H), H ** -0.5, dt, dev(), 12)
    b = torch.from_numpy(W.log_zipf_bias(E, 1.1)).to(dev()) if with_bias else None
    shape = abi.make_shape(num_tokens=T, hidden=H, num_experts=E, intermediate=64, top_k=min(2, E),
                           act_dtype=dt)
    ws = workspace(shape)
    lo = torch.empty(T, E, dtype=torch.float32, device=dev())
    ids = i32(T * shape.top_k)
    gates = f32(T * shape.top_k)
    abi.moe_route_topk(shape, x, wr, b, None, lo, None, ids, gates, ws)
    ref = oracle.router_logits(host(x), host(wr), None if b is None else b.cpu().numpy())
    assert_close_rms(lo.cpu().numpy(), ref, 1e-5, "logits")
