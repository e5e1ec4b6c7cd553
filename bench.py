"""Benchmark: one GPU's share of an expert-parallel MoE layer forward on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--experts bf16|mxfp8]
                    [--no-cpu-baseline]

A step is one moe_layer_forward call (router, top-k, dispatch, gather,
grouped gate/up + SwiGLU, grouped down, shared expert, combine) over one batch
of seeded synthetic input already resident in HBM.  The default workload is
the DeepSeek-V3-shaped layer, the largest of the workloads (T=8192, H=7168,
256 routed experts of I=2048 plus one shared expert, sigmoid scoring with
group-limited top-8, log-Zipf router bias; bf16 with fp32 accumulation).  With --experts mxfp8 the expert weights are
quantised once to MXFP8 before timing and each step is one
moe_layer_forward_mxfp8 call (routing on the bf16 x and router, x quantised
per token, scaled fp8 MFMA GEMMs, h re-quantised to MXFP8).  Prints one JSON
line on stdout.

Timing: W untimed warm-up steps; then up to five untimed steps with events
around every stage (moe_debug stage events) for the per-stage breakdown,
which picks the dominant grouped-GEMM stage; then the timed region: K steps
with a HIP event at every step boundary (per-step times: median and p95)
recorded on the stream the library launches on, and events around the
dominant stage only (two per step), which give its average duration for the
roofline figure.  The other workloads (--others) are measured the same way
with 10 steps each and summarised in the same line.  The CPU-oracle leg
times the plain CPU oracle on a bounded token sample of the headline
workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15      # MI355X dense bf16 MFMA
PEAK_FP8_FLOPS = 5.0e15       # MI355X dense fp8 MFMA
PEAK_F32_FLOPS = 157.3e12     # MI355X fp32 vector
PEAK_HBM = 8.0e12             # MI355X HBM3E bytes/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_model(cfg, counts_kept, eb):
    """Algorithmic flops and bytes of the grouped-GEMM stages from realized counts.
    eb: bytes per activation / weight element (2 for bf16, 1 + 1/32 for MXFP8:
    one code byte plus a 32nd of a scale byte); y and out are fp32."""
    H, I, Is, T = cfg.hidden, cfg.inter, cfg.shared_inter, cfg.tokens
    R = int(counts_kept.sum())
    touched = int((counts_kept > 0).sum())
    st = {}
    st["gate_up"] = dict(flops=4.0 * R * H * I,
                         bytes=R * H * eb + 2.0 * touched * I * H * eb + R * I * eb, units=R)
    st["down"] = dict(flops=2.0 * R * H * I, bytes=R * I * eb + 1.0 * touched * H * I * eb + R * H * 4.0, units=R)
    if Is:
        st["shared"] = dict(flops=6.0 * T * H * Is, bytes=T * H * eb + 3.0 * Is * H * eb + T * Is * eb * 2
                            + T * H * 4.0, units=T)
    return st


def cpu_baseline(cfg, inp, budget_s=15.0, mx=False):
    """The oracle as it stands, on a bounded token sample of the workload
    (its MXFP8 layer when mx, with the weights of the sample's experts
    quantised by the oracle outside the timed part)."""
    import oracle
    import workloads as W
    x, wr = W.to_numpy_raw(inp["x"]), W.to_numpy_raw(inp["w_router"])
    b, kpt = W.to_numpy_raw(inp["bias"]), W.to_numpy_raw(inp["k_per_token"])
    # routing of every token (capacity depends on all of them), timed alone
    t0 = time.perf_counter()
    lo = oracle.router_logits(x, wr, b)
    ids, _ = oracle.route(lo, cfg.top_k, kpt, cfg.score, cfg.renormalize, cfg.routed_scale, cfg.num_groups,
                          cfg.topk_groups, cfg.group_topn)
    t_route = time.perf_counter() - t0
    host = {k: W.to_numpy_raw(v) for k, v in inp.items() if k not in ("w_gate", "w_up", "w_down")}
    rng = np.random.default_rng(0)

    shared_q = None
    if mx and cfg.shared_inter:
        shared_q = {n: oracle.mxfp8_quantize(host[key])
                    for key, n in (("ws_gate", "gate"), ("ws_up", "up"), ("ws_down", "down"))}

    def run(n):
        tok = np.sort(rng.choice(cfg.tokens, size=n, replace=False)).astype(np.int32)
        used = sorted(set(int(e) for e in ids[tok].reshape(-1) if e >= 0))
        wq = {}
        for key in ("w_gate", "w_up", "w_down"):
            w = inp[key]
            arr = np.empty(tuple(w.shape), np.uint16 if cfg.dtype == W.DT_BF16 else np.float32)
            for e in used:
                arr[e] = W.to_numpy_raw(w[e])
            host[key] = arr
            if mx:
                c = np.zeros(arr.shape, np.uint8)
                sc = np.zeros(arr.shape[:-1] + (arr.shape[-1] // 32,), np.uint8)
                for e in used:
                    c[e], sc[e] = oracle.mxfp8_quantize(arr[e])
                wq[key[2:]] = (c, sc)
        t1 = time.perf_counter()
        if mx:
            oracle.layer_forward_mxfp8(host["x"], host["w_router"], wq, cfg.top_k, host["bias"],
                                       host["k_per_token"], cfg.score, cfg.renormalize, cfg.routed_scale,
                                       cfg.num_groups, cfg.topk_groups, cfg.group_topn, cfg.capacity_factor,
                                       shared_q, tokens=tok)
        else:
            oracle.layer_forward_cfg(cfg, host, tokens=tok)
        t_all = time.perf_counter() - t1
        return t_all

    n = min(cfg.tokens, 2 * oracle.num_threads())
    t_n = run(n)
    # the call re-routes every token; remove that, add back the sample's share
    per_tok = max(t_n - t_route, 1e-9) / n
    n2 = int(min(cfg.tokens, max(n, (budget_s - t_route) / per_tok)))
    if n2 > n:
        t_n = run(n2)
        n = n2
    t_sample = max(t_n - t_route, 1e-9) + t_route * n / cfg.tokens
    return dict(value=n / t_sample, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"{n} of {cfg.tokens} tokens of the {cfg.name} workload: routing of all tokens "
                       f"({t_route:.2f} s, charged pro rata) + per-token {'MXFP8 ' if mx else ''}FFN and "
                       f"combine of the sample ({t_n - t_route:.2f} s); fp64-accumulating C oracle, OpenMP "
                       f"over tokens")


def replica_leg(spec, cfg, shape, ws, step, hiprt, stream, K, torch, abi):
    """Times moe_map_replicas on this workload's routing (K calls between events)
    with EXTRA more copies of the HOT most loaded experts."""
    hot, extra = (int(v) for v in spec.split(":"))
    dev = torch.device("cuda:0")
    T, E, k = cfg.tokens, cfg.experts, cfg.top_k
    ids = torch.empty(T * k, dtype=torch.int32, device=dev)
    step(dict(topk_ids=ids))
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    counts = np.bincount(ids_h[ids_h >= 0], minlength=E)
    n = np.ones(E, np.int64)
    n[np.argsort(-counts, kind="stable")[:hot]] += extra
    off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    P = int(off[-1])
    rex = np.arange(P, dtype=np.int32)
    off_d, rex_d = torch.from_numpy(off).to(dev), torch.from_numpy(rex).to(dev)
    phys = torch.empty(T * k, dtype=torch.int32, device=dev)
    for _ in range(3):
        abi.moe_map_replicas(shape, ids, off_d, rex_d, P, phys, ws, stream=stream)
    a, b = hiprt.event_create(), hiprt.event_create()
    torch.cuda.synchronize()
    hiprt.event_record(a, stream)
    for _ in range(K):
        abi.moe_map_replicas(shape, ids, off_d, rex_d, P, phys, ws, stream=stream)
    hiprt.event_record(b, stream)
    torch.cuda.synchronize()
    us = hiprt.elapsed_ms(a, b) / K * 1e3
    ph = phys.cpu().numpy()
    pc = np.bincount(ph[ph >= 0], minlength=P)
    return {"hot_experts": hot, "extra_copies": extra, "physical_experts": P, "us_per_call": round(us, 2),
            "slots": int(T * k), "max_over_mean_logical": round(float(counts.max() / counts.mean()), 3),
            "max_over_mean_physical": round(float(pc.max() / pc.mean()), 3)}


def ep_leg(G, cfg, inp, ids, gates, K, torch, abi, hiprt, stream):
    """The expert-parallel exchange over G virtual ranks on this workload's
    routing: rows and bytes each rank would receive (one row per token and
    rank, against one row per routed slot without the per-rank merge), and
    the time of the send layout (with the payload gather) and of the
    source's combine of the returned rows, K calls each."""
    dev = torch.device("cuda:0")
    T, k, H = cfg.tokens, cfg.top_k, cfg.hidden
    shape = abi.make_shape(cfg)
    n_rows = T * min(k, G)
    ws = torch.empty(abi.moe_workspace_size(shape), dtype=torch.uint8, device=dev)
    i32 = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    rc, ro, st, sid, ssp = i32(G), i32(G + 1), i32(n_rows), i32(n_rows * k), i32(T * k)
    sg = torch.empty(max(n_rows * k, 1), dtype=torch.float32, device=dev)
    send_x = torch.empty(max(n_rows, 1), H, dtype=inp["x"].dtype, device=dev)
    partial = torch.randn(max(n_rows, 1), H, dtype=torch.float32, device=dev)
    out = torch.empty(T, H, dtype=torch.float32, device=dev)

    def layout():
        abi.moe_ep_dispatch_layout(shape, G, ids, gates, inp["x"], rc, ro, st, sid, sg, ssp, send_x, ws,
                                   stream=stream)

    def comb():
        abi.moe_ep_combine(shape, G, partial, ssp, None, out, stream=stream)

    res = {}
    for name, fn in (("layout_and_payload", layout), ("combine", comb)):
        for _ in range(3):
            fn()
        a, b = hiprt.event_create(), hiprt.event_create()
        torch.cuda.synchronize()
        hiprt.event_record(a, stream)
        for _ in range(K):
            fn()
        hiprt.event_record(b, stream)
        torch.cuda.synchronize()
        res[name + "_us"] = round(hiprt.elapsed_ms(a, b) / K * 1e3, 2)
    counts = rc.cpu().numpy()[:G]
    ids_h = ids.cpu().numpy()
    routed = int((ids_h >= 0).sum())
    eb = inp["x"].element_size()
    row_b = H * eb + k * 8                    # hidden row + the token's local ids and gates
    res.update({"ranks": G, "rows_sent": int(counts.sum()), "routed_slots": routed,
                "rows_per_rank": counts.tolist(),
                "max_over_mean_rank_rows": round(float(counts.max() / max(counts.mean(), 1e-9)), 3),
                "dispatch_bytes_per_rank": [int(c * row_b) for c in counts],
                "dispatch_bytes_total": int(counts.sum() * row_b),
                "dispatch_bytes_one_row_per_slot": int(routed * row_b),
                "combine_bytes_total_fp32": int(counts.sum() * H * 4),
                "layout_and_payload_GBps": round((T * H * eb + 2 * counts.sum() * row_b)
                                                 / (res["layout_and_payload_us"] * 1e-6) / 1e9, 1),
                "combine_GBps": round((counts.sum() * H * 4 + T * H * 4) / (res["combine_us"] * 1e-6) / 1e9, 1)})
    return res


def load_stats(cnt, kept):
    """Expert-load statistics of one layer call ("LLM MoE Expert Parallel
    production practice", step 1, the expert load metric set): routed slots
    per expert (before capacity), kept rows, drops, max/mean, the coefficient
    of variation and the experts that received no token."""
    cnt = np.asarray(cnt, np.float64)
    kept = np.asarray(kept, np.int64)
    mean = cnt.mean() if cnt.size else 0.0
    return {"rows_kept": int(kept.sum()), "dropped": int(cnt.sum() - kept.sum()),
            "experts_touched": int((kept > 0).sum()),
            "max_over_mean_load": round(float(cnt.max() / max(mean, 1e-9)), 3),
            "expert_load_cv": round(float(cnt.std() / max(mean, 1e-9)), 3),
            "zero_token_experts": int((cnt == 0).sum()),
            # experts by row count: in layers that mix big and small loads the
            # grouped GEMMs give experts below 128 kept rows 64-row tiles
            "experts_ge_128_rows": int((kept >= 128).sum()),
            "rows_in_experts_ge_128": int(kept[kept >= 128].sum()),
            "experts_1_to_127_rows": int(((kept > 0) & (kept < 128)).sum()),
            "rows_in_experts_1_to_127": int(kept[(kept > 0) & (kept < 128)].sum())}


def measure(cfg, K, warmup, mx, torch, abi, hiprt, W, replicas=None, ep_ranks=0, down_f16=True):
    """Runs the layer on cfg's seeded inputs: warm-up, a per-stage breakdown,
    then K timed steps with an event at every step boundary and events around
    the dominant grouped-GEMM stage.  down_f16 (bf16 layers): the down
    weights are converted to fp16 once, before timing (moe_convert_bf16_to_f16;
    the layer's results are bit-identical to converting inside every call).
    Returns (result dict, inputs)."""
    dev = torch.device("cuda:0")
    inp = W.make_layer_inputs(cfg, dev)
    down_f16 = down_f16 and not mx and cfg.dtype == W.DT_BF16
    shape = abi.make_shape(cfg, down_dtype=abi.MOE_F16 if down_f16 else 0)
    w_down, ws_down = inp["w_down"], inp["ws_down"]
    if down_f16:
        w_down = abi.to_f16_weights(inp["w_down"])
        ws_down = abi.to_f16_weights(inp["ws_down"]) if cfg.shared_inter else None
        torch.cuda.synchronize()
    if mx:
        mw = abi.mxfp8_ffn(inp["w_gate"], inp["w_up"], inp["w_down"], stream=None)
        mws = abi.mxfp8_ffn(inp["ws_gate"], inp["ws_up"], inp["ws_down"]) if cfg.shared_inter else None
        torch.cuda.synchronize()
        ws = torch.empty(abi.moe_workspace_size_mxfp8(shape), dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(abi.moe_workspace_size(shape), dtype=torch.uint8, device=dev)
    out = torch.empty(cfg.tokens, cfg.hidden, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    counts = torch.empty(cfg.experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(cfg.experts + 1, dtype=torch.int32, device=dev)
    dropped = torch.empty(1, dtype=torch.int32, device=dev)

    def step(dbg=None):
        if mx:
            abi.moe_layer_forward_mxfp8(shape, inp["x"], inp["w_router"], inp["bias"], inp["k_per_token"], mw, mws,
                                        out, dbg, ws, stream=stream)
        else:
            abi.moe_layer_forward(shape, inp["x"], inp["w_router"], inp["bias"], inp["k_per_token"],
                                  inp["w_gate"], inp["w_up"], w_down, inp["ws_gate"], inp["ws_up"],
                                  ws_down, out, dbg, ws, stream=stream)

    # one call with inspection outputs for the realized counts
    step(dict(expert_counts=counts, expert_offsets=offsets, num_dropped=dropped))
    torch.cuda.synchronize()
    kept = np.diff(offsets.cpu().numpy())
    cnt = counts.cpu().numpy()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    nst = len(abi.MOE_STAGES)
    eb = 1.0 + 1.0 / 32 if mx else cfg.elem_bytes
    model = gemm_model(cfg, kept, eb)

    def stage_dbg(stages):
        """MoeDebug whose timing events bracket the given stages only."""
        d = abi.MoeDebug()
        ev = {}
        for i in stages:
            ev[i] = (hiprt.event_create(), hiprt.event_create())
            d.stage_start[i], d.stage_stop[i] = ev[i]
        return d, ev

    # per-stage breakdown: a few untimed steps with events around every stage
    nb = min(K, 5)
    brk = [stage_dbg(range(nst)) for _ in range(nb)]
    for d, _ in brk:
        step(d)
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([hiprt.elapsed_ms(*ev[i]) for _, ev in brk]))
                for i, name in enumerate(abi.MOE_STAGES)}
    # dominant kernel: the grouped-GEMM stage with the largest time
    dom = max(model, key=lambda s: stage_ms[s])
    i_dom = abi.MOE_STAGES.index(dom)

    # timed region: K steps, an event at every step boundary (per-step times
    # for the median and p95) and events around the dominant stage
    timed = [stage_dbg([i_dom]) for _ in range(K)]
    bounds = [hiprt.event_create() for _ in range(K + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    hiprt.event_record(bounds[0], stream)
    for i, (d, _) in enumerate(timed):
        step(d)
        hiprt.event_record(bounds[i + 1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = hiprt.elapsed_ms(bounds[0], bounds[K])
    step_ms = np.array([hiprt.elapsed_ms(bounds[i], bounds[i + 1]) for i in range(K)])
    dom_ms = float(np.mean([hiprt.elapsed_ms(*ev[i_dom]) for _, ev in timed]))
    ms_per_step = total_ms / K

    peak_f = PEAK_FP8_FLOPS if mx else (PEAK_BF16_FLOPS if cfg.dtype == W.DT_BF16 else PEAK_F32_FLOPS)
    m = model[dom]
    t_s = dom_ms / 1e3
    bound = "mfma" if m["flops"] / peak_f >= m["bytes"] / PEAK_HBM else "hbm"
    if bound == "mfma":
        achieved, peak, unit = m["flops"] / t_s / 1e12, peak_f / 1e12, "TFLOP/s"
    else:
        achieved, peak, unit = m["bytes"] / t_s / 1e9, PEAK_HBM / 1e9, "GB/s"
    gemm_stages = [s for s in model]
    t_gemm = sum(stage_ms[s] for s in gemm_stages) / 1e3
    f_gemm = sum(model[s]["flops"] for s in gemm_stages)
    b_gemm = sum(model[s]["bytes"] for s in gemm_stages)
    t_roof_gemm = max(f_gemm / peak_f, b_gemm / PEAK_HBM)
    # the whole layer's bound from the realized counts: every grouped-GEMM
    # flop at the MFMA peak, or the weights of the touched experts, the
    # router, x in and the fp32 output once at the HBM peak
    es = cfg.elem_bytes if not mx else eb
    f_layer = f_gemm + 2.0 * cfg.tokens * cfg.hidden * cfg.experts
    b_layer = (es * (3.0 * cfg.hidden * cfg.inter * int((kept > 0).sum()) + 3.0 * cfg.hidden * cfg.shared_inter
                     + cfg.experts * cfg.hidden) + cfg.tokens * cfg.hidden * (cfg.elem_bytes + 4.0))
    t_roof_layer = max(f_layer / peak_f, b_layer / PEAK_HBM)

    res = dict(down_f16=down_f16, ms_per_step=ms_per_step, tokens_per_s=cfg.tokens / (ms_per_step / 1e3), wall=wall,
               step_ms=step_ms, stage_ms=stage_ms, dom=dom, dom_ms=dom_ms, bound=bound, achieved=achieved,
               peak=peak, unit=unit, model=model, t_gemm=t_gemm, f_gemm=f_gemm, b_gemm=b_gemm,
               t_roof_gemm=t_roof_gemm, peak_f=peak_f, t_roof_layer=t_roof_layer, f_layer=f_layer,
               b_layer=b_layer, load=load_stats(cnt, kept))
    if replicas:
        res["replica_map"] = replica_leg(replicas, cfg, shape, ws, step, hiprt, stream, K, torch, abi)
    if ep_ranks and cfg.experts % ep_ranks == 0:
        ids = torch.empty(cfg.tokens * cfg.top_k, dtype=torch.int32, device=dev)
        gates = torch.empty(cfg.tokens * cfg.top_k, dtype=torch.float32, device=dev)
        step(dict(topk_ids=ids, topk_gates=gates))
        torch.cuda.synchronize()
        res["ep_exchange"] = ep_leg(ep_ranks, cfg, inp, ids, gates, K, torch, abi, hiprt, stream)
    return res, inp


def summary_of(cfg, r):
    """One workload's figures for the all-workloads table of the line."""
    return {"tokens": cfg.tokens, "ms_per_step": round(r["ms_per_step"], 4),
            "tokens_per_s": round(r["tokens_per_s"], 1),
            "p50_ms": round(float(np.median(r["step_ms"])), 4),
            "p95_ms": round(float(np.percentile(r["step_ms"], 95)), 4),
            "layer_frac_of_roofline": round(r["t_roof_layer"] / (r["ms_per_step"] / 1e3), 4),
            "grouped_gemm_frac_of_roofline": round(r["t_roof_gemm"] / r["t_gemm"], 4),
            "dominant_kernel": r["dom"], "dominant_bound": r["bound"],
            "dominant_frac_of_peak": round(r["achieved"] / r["peak"], 4),
            "max_over_mean_load": r["load"]["max_over_mean_load"],
            "expert_load_cv": r["load"]["expert_load_cv"],
            "zero_token_experts": r["load"]["zero_token_experts"]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="deepseek_v3")
    ap.add_argument("--experts", choices=("bf16", "mxfp8"), default="bf16",
                    help="expert weight format: the workload's bf16, or MXFP8 (E4M3 codes, one E8M0 scale "
                         "per 32 elements) quantised once before timing")
    ap.add_argument("--down-weights", choices=("f16", "bf16"), default="f16",
                    help="bf16 layers: down weights converted to fp16 once before timing (f16; the same "
                         "products as the conversion inside every call), or passed as bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--others", default="tiny_fp32,mixtral_prefill,mixtral_decode,qwen3_skewed",
                    help="comma-separated workloads also measured in the same run (10 steps each) and "
                         "summarised under 'all_workloads'; 'none' for none")
    ap.add_argument("--ep-ranks", type=int, default=8,
                    help="also lay out the dispatch exchange of this workload's routing over this many "
                         "virtual expert-parallel ranks (contiguous expert blocks) and time the layout and the "
                         "source's combine; 0: skip")
    ap.add_argument("--replicas", default=None, metavar="HOT:EXTRA",
                    help="also time the redundant-expert routing step (moe_map_replicas) with EXTRA more "
                         "copies of the HOT most loaded experts, and report the load balance it gives")
    ap.add_argument("--set", action="append", default=[], metavar="FIELD=VALUE",
                    help="override a field of the workload's layer shape (e.g. top_k=8, k_choices=none, "
                         "capacity_factor=0); the overrides are echoed in the config; the seeds stay those "
                         "of the named workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device-to-device copy first (a kernel of known HBM traffic "
                         "for scaling profiler byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the layer share it measures is "
                                   "one GPU's expert-parallel share; multi-GPU runs are not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import workloads as W
    from expert_serving_amd import abi, hiprt

    cfg = W.CONFIGS[args.workload]
    overrides = {}
    for item in args.set:
        key, val = item.split("=", 1)
        cur = getattr(cfg, key)
        if val.lower() == "none":
            v = None
        elif key == "k_choices":
            v = tuple(int(c) for c in val.split(","))
        else:
            v = type(cur)(float(val)) if isinstance(cur, (int, float)) and not isinstance(cur, bool) else val
        overrides[key] = v
    if overrides:
        cfg = cfg.replace(**overrides)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    mx = args.experts == "mxfp8"
    if mx and cfg.dtype != W.DT_BF16:
        print(json.dumps({"error": "MXFP8 experts need a bf16 workload"}))
        sys.exit(2)

    f16 = args.down_weights == "f16"
    r, inp = measure(cfg, args.steps, args.warmup, mx, torch, abi, hiprt, W, args.replicas, args.ep_ranks, f16)
    K = args.steps
    dom, m = r["dom"], r["model"][r["dom"]]

    # HBM traffic of the dominant kernel from the committed counter summary,
    # only while the kernel source is the one the counters were taken on
    from expert_serving_amd import profiling
    traffic = None
    rec = profiling.read_traffic(os.path.join(ROOT, "profiles",
                                              f"{dom}_gemm_{'mxfp8_' if mx else ''}{cfg.name}_traffic.md"))
    if rec and rec.get("source_sha256") == profiling.source_sha256():
        traffic = float(rec["traffic_bytes"])

    line = {
        "metric": "MoE-layer tokens/sec at 1 GPU; grouped-GEMM % of bf16 MFMA / HBM peak",
        "value": round(r["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 (MXFP8 experts; bf16 router)" if mx else ("bf16" if cfg.dtype == W.DT_BF16 else "f32"),
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
        "config": {"workload": cfg.name, "tokens": cfg.tokens, "hidden": cfg.hidden, "experts": cfg.experts,
                   "top_k": cfg.top_k, "intermediate": cfg.inter, "shared_intermediate": cfg.shared_inter,
                   "capacity_factor": cfg.capacity_factor, "parallelism": "one GPU's expert-parallel share",
                   "expert_format": args.experts,
                   "down_weights": "f16 (converted once before timing)" if r["down_f16"] else
                   ("mxfp8" if mx else ("bf16" if cfg.dtype == W.DT_BF16 else "f32")),
                   **({"overrides": {k: v for k, v in overrides.items()}} if overrides else {})},
        "roofline": {"bound": r["bound"], "achieved": round(r["achieved"], 2), "peak": r["peak"], "unit": r["unit"],
                     "frac": round(r["achieved"] / r["peak"], 4), "traffic": traffic, "kernel": dom,
                     "kernel_ms": round(r["dom_ms"], 4),
                     "per_launch_algorithmic": {"flops": m["flops"], "bytes": m["bytes"], "rows": m["units"]}},
        # per-step latency over the K timed steps (events at every step boundary)
        "latency_ms": {"p50": round(float(np.median(r["step_ms"])), 4),
                       "p95": round(float(np.percentile(r["step_ms"], 95)), 4),
                       "min": round(float(r["step_ms"].min()), 4), "max": round(float(r["step_ms"].max()), 4)},
        "layer_roofline": {"ms": round(r["t_roof_layer"] * 1e3, 4), "flops": r["f_layer"], "bytes": r["b_layer"],
                           "frac": round(r["t_roof_layer"] / (r["ms_per_step"] / 1e3), 4)},
        "grouped_gemm": {"ms": round(r["t_gemm"] * 1e3, 4), "tflops": round(r["f_gemm"] / r["t_gemm"] / 1e12, 2),
                         "frac_of_roofline": round(r["t_roof_gemm"] / r["t_gemm"], 4),
                         "frac_of_mfma_peak": round(r["f_gemm"] / r["t_gemm"] / r["peak_f"], 4),
                         "mfma_peak_tflops": r["peak_f"] / 1e12,
                         "frac_of_hbm_peak": round(r["b_gemm"] / r["t_gemm"] / PEAK_HBM, 4)},
        # from the separate breakdown steps (events around every stage)
        "stages_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()},
        "routing": r["load"],
        "host_wall_s": round(r["wall"], 3),
    }
    if "replica_map" in r:
        line["replica_map"] = r["replica_map"]
    if "ep_exchange" in r:
        line["ep_exchange"] = r["ep_exchange"]
    others = [] if args.others.lower() == "none" else [o for o in args.others.split(",") if o and o != cfg.name]
    if others:
        allw = {cfg.name: summary_of(cfg, r)}
        for name in others:
            oc = W.CONFIGS[name]
            log(f"measuring {name} ...")
            ro, _ = measure(oc, 10, 2, mx and oc.dtype == W.DT_BF16, torch, abi, hiprt, W, down_f16=f16)
            allw[name] = summary_of(oc, ro)
            torch.cuda.empty_cache()
        line["all_workloads"] = allw
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_budget, mx=mx)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
