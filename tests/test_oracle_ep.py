"""Pins of the oracle's expert-parallel exchange layout and combine (CPU only).

"Expert Parallelism: MoE model parallel split": experts in G contiguous
blocks, one per rank (§8, the EP=8 layout of 256 experts); two exchanges per
layer, dispatch and combine (§3, §12 Q2); rows bound for one rank grouped
together (§7 and §12, token sorting).  "Expert parallelism for MoE serving",
deployment examples: node-limited routing bounds the ranks a token's experts
span, so a token travels once to each such rank.  Each pin checks the oracle
against library routines (bincount, cumsum, lexsort), closed forms, a
hand-worked example, the special cases G = 1 and G = E (where the layout
reduces to the single-GPU dispatch permutation), and the whole exchange
chain against the oracle's layer.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def random_routing(T, E, k, seed, unused=0.1):
    """Distinct expert ids per token in descending-logit slot order, some
    slots unused (-1, at the end as routing writes them), gates in (0, 1]."""
    rng = np.random.default_rng(seed)
    ids = np.full((T, k), -1, np.int32)
    gates = np.zeros((T, k), np.float32)
    for t in range(T):
        kt = k if rng.random() > unused else int(rng.integers(0, k))
        ids[t, :kt] = rng.choice(E, size=kt, replace=False)
        gates[t, :kt] = rng.random(kt).astype(np.float32) + 1e-3
    return ids, gates


def library_layout(ids, gates, E, G):
    """The same layout from numpy: (rank, token) pairs by lexsort, counts by
    bincount, offsets by cumsum."""
    T, k = ids.shape
    epr = E // G
    valid = ids >= 0
    rank = np.where(valid, ids // epr, -1)
    pairs = sorted({(int(rank[t, j]), t) for t in range(T) for j in range(k) if valid[t, j]})
    d_of = np.array([p[0] for p in pairs], np.int64)
    t_of = np.array([p[1] for p in pairs], np.int64)
    order = np.lexsort((t_of, d_of))
    d_of, t_of = d_of[order], t_of[order]
    counts = np.bincount(d_of, minlength=G)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    return d_of, t_of, counts, offsets


@pytest.mark.parametrize("T,E,k,G", [(37, 8, 2, 4), (100, 16, 4, 4), (64, 32, 8, 8), (5, 8, 3, 8), (300, 64, 6, 16),
                                     (1, 8, 2, 2)])
def test_layout_matches_library_routines(T, E, k, G):
    ids, gates = random_routing(T, E, k, seed=T + E + k + G)
    L = oracle.ep_layout(ids, gates, E, G)
    d_of, t_of, counts, offsets = library_layout(ids, gates, E, G)
    assert np.array_equal(L["rank_counts"], counts)
    assert np.array_equal(L["rank_offsets"], offsets)
    S = L["S"]
    assert S == len(t_of) == offsets[-1]
    assert np.array_equal(L["send_token"][:S], t_of)
    n_rows = T * min(k, G)
    assert np.all(L["send_token"][S:] == -1) and np.all(L["send_ids"][S:] == -1) and np.all(L["send_gates"][S:] == 0)
    epr = E // G
    for p in range(S):
        t, d = t_of[p], d_of[p]
        on = (ids[t] >= 0) & (ids[t] // epr == d)
        assert np.array_equal(L["send_ids"][p], np.where(on, ids[t] - d * epr, -1))
        assert np.array_equal(L["send_gates"][p], np.where(on, gates[t], 0))
    for t in range(T):
        for j in range(k):
            p = L["slot_send_pos"][t, j]
            if ids[t, j] < 0:
                assert p == -1
            else:
                assert L["send_token"][p] == t and d_of[p] == ids[t, j] // epr
    # every row carries at least one slot, and a token's rows sit on distinct ranks
    assert np.all((L["send_ids"][:S] >= 0).any(1))
    assert n_rows >= S


def test_one_expert_per_rank_is_the_dispatch_permutation():
    """G = E: every rank holds one expert and a token's slots hit distinct
    ranks, so the layout is the single-GPU dispatch (no capacity): counts,
    offsets, the position of every slot and the token of every row."""
    T, E, k = 200, 16, 4
    ids, gates = random_routing(T, E, k, seed=3)
    L = oracle.ep_layout(ids, gates, E, E)
    d = oracle.dispatch(ids, E)
    assert np.array_equal(L["rank_counts"], d["counts"])
    assert np.array_equal(L["rank_offsets"], d["offsets"])
    assert np.array_equal(L["slot_send_pos"], d["row_of_slot"])
    assert np.array_equal(L["send_token"][:L["S"]], d["row_token"][:d["R"]])
    assert np.all(L["send_ids"][:L["S"]].max(1) == 0)       # local id 0 on every rank


def test_single_rank_is_one_row_per_routed_token():
    T, E, k = 50, 8, 2
    ids, gates = random_routing(T, E, k, seed=4, unused=0.3)
    L = oracle.ep_layout(ids, gates, E, 1)
    routed = np.nonzero((ids >= 0).any(1))[0]
    assert L["S"] == len(routed)
    assert np.array_equal(L["send_token"][:L["S"]], routed)
    assert np.array_equal(L["send_ids"][:L["S"]], ids[routed])
    assert np.array_equal(L["send_gates"][:L["S"]], np.where(ids[routed] >= 0, gates[routed], 0))


def test_group_limited_routing_bounds_rows_per_token():
    """With G ranks equal to the routing groups (the EP=8 layout of 256
    experts), a token spans at most topk_groups ranks: at most T*topk_groups
    rows instead of T*k per-expert copies."""
    layout = json.load(open(os.path.join(GOLDEN, "ep8_expert_layout.json")))
    G = layout["num_gpus"]
    cfg = W.CONFIGS["deepseek_v3"].with_tokens(512)
    assert cfg.experts == layout["num_experts"]
    rng = np.random.default_rng(9)
    logits = (rng.standard_normal((cfg.tokens, cfg.experts)) + W.log_zipf_bias(cfg.experts, cfg.zipf_s)).astype(np.float32)
    ids, gates = oracle.route(logits, cfg.top_k, None, cfg.score, cfg.renormalize, cfg.routed_scale, cfg.num_groups,
                              cfg.topk_groups, cfg.group_topn)
    L = oracle.ep_layout(ids, gates, cfg.experts, G)
    per_token = np.bincount(L["send_token"][:L["S"]], minlength=cfg.tokens)
    assert per_token.max() <= cfg.topk_groups
    assert L["S"] <= cfg.tokens * cfg.topk_groups < cfg.tokens * cfg.top_k
    # the ranks a token reaches are exactly its kept groups
    epr = cfg.experts // G
    for t in range(0, cfg.tokens, 17):
        rows = np.nonzero(L["send_token"][:L["S"]] == t)[0]
        ranks = np.searchsorted(L["rank_offsets"], rows, side="right") - 1
        assert sorted(ranks.tolist()) == sorted(set((ids[t] // epr).tolist()))


def test_hand_worked_layout_and_combine():
    """E = 8 experts on G = 4 ranks (experts 2d, 2d+1 on rank d), k = 3.
    token 0: experts 5, 0, 1 -> ranks 2, 0, 0
    token 1: experts 2, 3, 6 -> ranks 1, 1, 3
    token 2: experts 7, unused, unused -> rank 3
    Rows: rank 0: token 0; rank 1: token 1; rank 2: token 0; rank 3: tokens 1, 2."""
    ids = np.array([[5, 0, 1], [2, 3, 6], [7, -1, -1]], np.int32)
    gates = np.array([[0.5, 0.3, 0.2], [0.6, 0.3, 0.1], [1.0, 0.0, 0.0]], np.float32)
    L = oracle.ep_layout(ids, gates, 8, 4)
    assert L["rank_counts"].tolist() == [1, 1, 1, 2]
    assert L["rank_offsets"].tolist() == [0, 1, 2, 3, 5]
    assert L["send_token"].tolist() == [0, 1, 0, 1, 2, -1, -1, -1, -1]
    assert L["send_ids"][:5].tolist() == [[-1, 0, 1], [0, 1, -1], [1, -1, -1], [-1, -1, 0], [1, -1, -1]]
    assert np.allclose(L["send_gates"][:5], [[0, .3, .2], [.6, .3, 0], [.5, 0, 0], [0, 0, .1], [1, 0, 0]])
    assert L["slot_send_pos"].tolist() == [[2, 0, 0], [1, 1, 3], [4, -1, -1]]
    # combine: token 0 sums rows 0 and 2, token 1 rows 1 and 3, token 2 row 4
    partial = np.arange(5 * 2, dtype=np.float32).reshape(5, 2)
    out = oracle.ep_combine(partial, L["slot_send_pos"])
    assert out.tolist() == [[0 + 4, 1 + 5], [2 + 6, 3 + 7], [8, 9]]
    ys = np.full((3, 2), 0.5, np.float32)
    assert np.array_equal(oracle.ep_combine(partial, L["slot_send_pos"], ys), out + 0.5)


def test_combine_matches_sparse_matmul():
    T, E, k, G, H = 60, 16, 4, 4, 24
    ids, gates = random_routing(T, E, k, seed=8, unused=0.2)
    L = oracle.ep_layout(ids, gates, E, G)
    rng = np.random.default_rng(1)
    partial = rng.standard_normal((T * min(k, G), H)).astype(np.float32)
    ys = rng.standard_normal((T, H)).astype(np.float32)
    out = oracle.ep_combine(partial, L["slot_send_pos"], ys)
    S = np.zeros((T, partial.shape[0]))
    for p in range(L["S"]):
        S[L["send_token"][p], p] = 1.0
    ref = S @ partial.astype(np.float64) + ys
    assert np.abs(out - ref).max() <= 1e-6 * np.sqrt((ref ** 2).mean())


def _rank_chain(x, ids, gates, wg, wu, wd, G, ws=None):
    """The exchange over G ranks with the oracle's step functions: layout,
    then on every rank its received rows through a local dispatch (local
    expert ids), its own experts' FFN and a combine per received row (the
    pre-reduced partial sums), then the source's sum over ranks."""
    T = x.shape[0]
    E = wg.shape[0]
    epr = E // G
    L = oracle.ep_layout(ids, gates, E, G)
    H = x.shape[1]
    partial = np.zeros((max(len(L["send_token"]), 1), H), np.float32)
    for d in range(G):
        a, b = L["rank_offsets"][d], L["rank_offsets"][d + 1]
        if a == b:
            continue
        rid = L["send_ids"][a:b]
        disp = oracle.dispatch(rid, epr)
        xr = x[L["send_token"][a:b]]
        xp = xr[disp["row_token"][:disp["R"]]]
        y = oracle.grouped_ffn(xp, disp["offsets"], wg[d * epr:(d + 1) * epr], wu[d * epr:(d + 1) * epr],
                               wd[d * epr:(d + 1) * epr])
        partial[a:b] = oracle.combine(y if len(y) else np.zeros((1, H), np.float32), disp["row_of_slot"],
                                      L["send_gates"][a:b])
    ys = None
    if ws is not None:
        ys = oracle.grouped_ffn(x, np.array([0, T], np.int32), *(w[None] for w in ws))
    return oracle.ep_combine(partial, L["slot_send_pos"], ys), L


@pytest.mark.parametrize("G,shared", [(1, False), (2, False), (4, True), (8, False)])
def test_exchange_chain_equals_the_layer(G, shared):
    """Layout -> per-rank local dispatch, FFN and pre-reduced combine -> the
    source's sum over ranks gives the oracle layer's output (fp64 sums in
    another order: within 1e-6 of the RMS)."""
    rng = np.random.default_rng(20 + G)
    T, H, E, I, k = 40, 32, 8, 48, 3
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (rng.standard_normal((E, H)) / math.sqrt(H)).astype(np.float32)
    wg = (rng.standard_normal((E, I, H)) / math.sqrt(H)).astype(np.float32)
    wu = (rng.standard_normal((E, I, H)) / math.sqrt(H)).astype(np.float32)
    wd = (rng.standard_normal((E, H, I)) / math.sqrt(I)).astype(np.float32)
    sh = None
    if shared:
        sh = ((rng.standard_normal((I, H)) / math.sqrt(H)).astype(np.float32),
              (rng.standard_normal((I, H)) / math.sqrt(H)).astype(np.float32),
              (rng.standard_normal((H, I)) / math.sqrt(I)).astype(np.float32))
    ref = oracle.layer_forward(x, wr, wg, wu, wd, k, ws_gate=sh[0] if sh else None, ws_up=sh[1] if sh else None,
                               ws_down=sh[2] if sh else None)
    out, L = _rank_chain(x, ref["ids"], ref["gates"], wg, wu, wd, G, sh)
    r = np.sqrt((ref["out"].astype(np.float64) ** 2).mean())
    assert np.abs(out - ref["out"]).max() <= 1e-6 * r
    # dedup: rows sent = distinct (token, rank) pairs <= routed slots
    assert L["S"] <= int((ref["ids"] >= 0).sum())
    if G == E:
        assert L["S"] == int((ref["ids"] >= 0).sum())


def test_rank_of_each_expert_is_the_pages_ep8_layout():
    """One token routed to expert e alone lands on the rank whose block the
    EP=8 layout printed on the page assigns to e."""
    layout = json.load(open(os.path.join(GOLDEN, "ep8_expert_layout.json")))
    E, G = layout["num_experts"], layout["num_gpus"]
    ids = np.arange(E, dtype=np.int32)[:, None]
    gates = np.ones((E, 1), np.float32)
    L = oracle.ep_layout(ids, gates, E, G)
    for d, (lo, hi) in enumerate(layout["gpu_expert_ranges"]):
        rows = np.arange(L["rank_offsets"][d], L["rank_offsets"][d + 1])
        assert L["send_token"][rows].tolist() == list(range(lo, hi + 1))
        assert L["send_ids"][rows, 0].tolist() == list(range(hi - lo + 1))
