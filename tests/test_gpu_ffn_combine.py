"""GPU parity of the grouped SwiGLU FFN (S7-S8) and the combine (S10) through
the C ABI against the CPU oracle.

Tolerances: bf16 inputs with fp32 accumulation, h rounded to fp16:
max|err| <= 2e-2 * RMS(reference); fp32 layers: 1e-4 * RMS; combine (fp32
arithmetic on fp32 inputs): 1e-5 * RMS.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from expert_serving_amd import abi

from gpu_util import assert_close_rms, dev, host, say, workspace

pytestmark = pytest.mark.gpu

FFN_CASES = [
    # name, dtype, E, H, I, rows per expert, tokens*k (sets the tile plan)
    ("bf16_big_tiles", W.DT_BF16, 4, 512, 384, [300, 0, 77, 129], 4096),
    ("bf16_small_tiles", W.DT_BF16, 8, 1024, 640, [16, 3, 0, 40, 17, 1, 64, 9], 150),
    ("bf16_one_expert_ragged", W.DT_BF16, 1, 256, 192, [203], 203),
    ("bf16_many_experts_skew", W.DT_BF16, 64, 256, 128, None, 4096),
    # odd numbers of 64-wide K stages in both projections (5 and 3), all 256-row tiles
    ("bf16_odd_k_stages", W.DT_BF16, 2, 320, 192, [600, 300], 1024),
    # the smallest K (one 64-wide stage), a big and an empty expert
    ("bf16_min_k", W.DT_BF16, 2, 64, 64, [300, 0], 600),
    # no small expert: the remainders past the last full 256-row tile (44, 1
    # and 40 rows) ride on 64-row tiles beside the big ones
    ("bf16_big_tiles_with_tails", W.DT_BF16, 3, 512, 384, [300, 257, 552], 4096),
    # a token or two: two one-row experts, so the gate/up K is split into
    # parts that a separate kernel adds before SwiGLU
    ("bf16_two_rows_split_gate_up", W.DT_BF16, 8, 1024, 512, [1, 0, 0, 0, 0, 0, 1, 0], 2),
    # big and small experts in one interleaved launch, the small ones with
    # 1, 2, 3 and 4 rows (vector-ALU tiles of 1, 2 and 4 token rows) and 5
    # rows (MFMA); 17 and 10 K segments (pipeline remainders); the last
    # column tile of each projection partly past N
    ("bf16_skinny_small_experts", W.DT_BF16, 8, 1088, 640, [700, 1, 2, 3, 4, 5, 0, 300], 1015),
    ("f32_tiny", W.DT_F32, 3, 128, 96, [40, 0, 33], 73),
    ("f32_ragged", W.DT_F32, 5, 64, 36, [1, 31, 32, 33, 70], 167),
]


@pytest.mark.parametrize("name,dt,E,H,I,rows,slots", FFN_CASES, ids=[c[0] for c in FFN_CASES])
def test_grouped_ffn_parity(name, dt, E, H, I, rows, slots):
    say(f"ffn case {name}")
    if rows is None:
        rng = np.random.default_rng(4)
        p = np.arange(1, E + 1, dtype=np.float64) ** -1.2
        rows = rng.multinomial(slots, p / p.sum()).tolist()
    R = sum(rows)
    offsets = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    # T*k sets the buffers and the tile plan; R <= T*k
    shape = abi.make_shape(num_tokens=slots, hidden=H, num_experts=E, intermediate=I, top_k=1, act_dtype=dt)
    x = W.normal((slots, H), 1.0, dt, dev(), 21)
    wg = W.normal((E, I, H), H ** -0.5, dt, dev(), 22)
    wu = W.normal((E, I, H), H ** -0.5, dt, dev(), 23)
    wd = W.normal((E, H, I), I ** -0.5, dt, dev(), 24)
    y = torch.full((slots, H), float("nan"), dtype=torch.float32, device=dev())
    ws = workspace(shape)
    abi.moe_grouped_ffn(shape, x, torch.from_numpy(offsets).to(dev()), wg, wu, wd, y, ws)
    torch.cuda.synchronize()
    ref = oracle.grouped_ffn(host(x)[:R], offsets, host(wg), host(wu), host(wd))
    tol = 2e-2 if dt == W.DT_BF16 else 1e-4
    assert_close_rms(y[:R].cpu().numpy(), ref, tol, name)
    # rows past R are not written
    if R < slots:
        assert torch.isnan(y[R:]).all()


@pytest.mark.parametrize("out_bf16", [False, True])
def test_combine_parity(out_bf16):
    T, E, k, H = 777, 9, 3, 512
    ids, gates = oracle.route(W.make_logits(T, E, seed=31).numpy(), k)
    d = oracle.dispatch(ids, E, 0.8)
    R = d["R"]
    g = torch.Generator().manual_seed(5)
    y = torch.randn(T * k, H, generator=g)
    ys = torch.randn(T, H, generator=g)
    shape = abi.make_shape(num_tokens=T, hidden=H, num_experts=E, intermediate=64, top_k=k,
                           out_dtype=abi.MOE_BF16 if out_bf16 else abi.MOE_F32)
    out = torch.empty(T, H, dtype=torch.bfloat16 if out_bf16 else torch.float32, device=dev())
    abi.moe_combine(shape, y.to(dev()), torch.from_numpy(d["row_of_slot"]).to(dev()),
                    torch.from_numpy(gates).to(dev()), ys.to(dev()), out)
    ref = oracle.combine(y[:R].numpy(), d["row_of_slot"], gates, ys.numpy())
    got = out.float().cpu().numpy()
    if out_bf16:
        # one bf16 rounding of the fp32 sum
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
    else:
        assert_close_rms(got, ref, 1e-5, "combine")
    # without the shared expert
    out2 = torch.empty(T, H, dtype=torch.float32, device=dev())
    shape.out_dtype = abi.MOE_F32
    abi.moe_combine(shape, y.to(dev()), torch.from_numpy(d["row_of_slot"]).to(dev()),
                    torch.from_numpy(gates).to(dev()), None, out2)
    assert_close_rms(out2.cpu().numpy(), oracle.combine(y[:R].numpy(), d["row_of_slot"], gates), 1e-5, "combine")
