"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks one oracle function against a library routine, a closed form,
brute force on tiny inputs, an invariant the pages state, or a hand-worked
example, chosen so that a dropped term, a wrong sign or index, or a transposed
operand fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy import special

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(20261203)


def f32(x):
    return np.float32(x)


def rand_bf16(shape, std, rng):
    a = (rng.standard_normal(shape) * std).astype(np.float32)
    bits = a.view(np.uint32)
    # round to nearest even into the upper 16 bits
    rounding = ((bits >> 16) & 1) + 0x7FFF
    return ((bits + rounding) >> 16).astype(np.uint16)


def widen(a):
    return W.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


# ---------------------------------------------------------------------------
# router logits
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bf16", [False, True])
def test_router_logits_match_float64_matmul(bf16):
    T, H, E = 37, 96, 5
    if bf16:
        x = rand_bf16((T, H), 1.0, RNG)
        wr = rand_bf16((E, H), 1 / math.sqrt(H), RNG)
    else:
        x = RNG.standard_normal((T, H)).astype(np.float32)
        wr = (RNG.standard_normal((E, H)) / math.sqrt(H)).astype(np.float32)
    b = RNG.standard_normal(E).astype(np.float32)
    got = oracle.router_logits(x, wr, b)
    ref = (widen(x).astype(np.float64) @ widen(wr).astype(np.float64).T + b).astype(np.float32)
    # both are the fp64 result rounded once: equal up to one ulp
    ulp = np.spacing(np.abs(ref))
    assert np.all(np.abs(got - ref) <= ulp)
    # and the bias really enters
    got0 = oracle.router_logits(x, wr, None)
    assert np.allclose(got - got0, b[None, :], atol=1e-5)


# ---------------------------------------------------------------------------
# sigmoid_spec
# ---------------------------------------------------------------------------
def test_sigmoid_spec_accuracy_and_special_values():
    xs = np.concatenate([
        np.linspace(-30, 30, 2_000_001, dtype=np.float32),
        RNG.standard_normal(200_000).astype(np.float32) * 4,
        np.array([-1e-30, 1e-30, -0.0, 0.0, 1e-7, -1e-7], np.float32),
    ])
    y = oracle.sigmoid_spec(xs)
    ref = 1.0 / (1.0 + np.exp(-xs.astype(np.float64)))
    err_ulp = np.abs(y.astype(np.float64) - ref) / np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert err_ulp.max() <= 3.0, err_ulp.max()
    assert oracle.sigmoid_spec(np.array([0.0], np.float32))[0] == np.float32(0.5)
    # clamping: beyond +-30 the value is the value at +-30
    far = oracle.sigmoid_spec(np.array([-100, -30, 30, 100, 1e30, -1e30], np.float32))
    assert far[0] == far[1] and far[2] == far[3] == far[4] and far[5] == far[1]
    # monotone non-decreasing on a sorted grid
    grid = np.linspace(-30, 30, 100_001, dtype=np.float32)
    assert np.all(np.diff(oracle.sigmoid_spec(grid)) >= 0)
    # symmetry of the logistic function within rounding: s(x) + s(-x) = 1
    a = np.linspace(-10, 10, 10001, dtype=np.float32)
    s = oracle.sigmoid_spec(a).astype(np.float64) + oracle.sigmoid_spec(-a).astype(np.float64)
    assert np.abs(s - 1).max() < 3e-7


# ---------------------------------------------------------------------------
# selection and gates
# ---------------------------------------------------------------------------
def stable_topk(l, k):
    """Library selection: stable argsort of the negated logits keeps the lower
    expert index first among equal logits."""
    return np.argsort(-l, kind="stable")[:k]


@pytest.mark.parametrize("E,k", [(8, 2), (8, 8), (16, 3), (256, 8), (128, 8), (5, 1), (64, 16)])
def test_plain_topk_matches_stable_argsort_with_ties(E, k):
    T = 300
    l = W.make_logits(T, E, seed=E * 31 + k, tie_fraction=0.3).numpy()
    ids, gates = oracle.route(l, k)
    for t in range(T):
        assert list(ids[t]) == list(stable_topk(l[t], k)), t
    # ids distinct and in range
    assert np.all((ids >= 0) & (ids < E))
    assert all(len(set(r)) == k for r in ids.tolist())
    # gates: softmax over the selected logits (the renormalised full softmax)
    for t in range(T):
        ref = special.softmax(l[t, ids[t]].astype(np.float64))
        assert np.allclose(gates[t], ref, rtol=2e-7, atol=1e-30)
    assert np.allclose(gates.sum(1), 1.0, atol=1e-6)


def test_exhaustive_no_better_unselected_expert():
    # brute force on tiny E: no unselected expert outranks a selected one
    rng = np.random.default_rng(7)
    for E in (1, 2, 3, 4, 6):
        for k in range(1, E + 1):
            l = rng.integers(-2, 3, size=(200, E)).astype(np.float32)   # many exact ties
            ids, _ = oracle.route(l, k)
            for t in range(200):
                sel = set(ids[t].tolist())
                for e in range(E):
                    if e in sel:
                        continue
                    for s in sel:
                        assert (l[t, s] > l[t, e]) or (l[t, s] == l[t, e] and s < e)
                # slot order: descending logit, ties by lower index
                for j in range(k - 1):
                    a, b = ids[t, j], ids[t, j + 1]
                    assert l[t, a] > l[t, b] or (l[t, a] == l[t, b] and a < b)


def test_softmax_without_renorm_is_full_softmax():
    l = W.make_logits(50, 8, seed=3).numpy()
    ids, gates = oracle.route(l, 8, renorm=0)
    for t in range(50):
        p = special.softmax(l[t].astype(np.float64))
        assert np.allclose(gates[t], p[ids[t]], rtol=2e-7)
    ids2, gates2 = oracle.route(l, 2, renorm=0)
    for t in range(50):
        p = special.softmax(l[t].astype(np.float64))
        assert np.allclose(gates2[t], p[ids2[t]], rtol=2e-7)
        assert gates2[t].sum() < 1.0


def test_sigmoid_gates_renormalised_and_scaled():
    l = W.make_logits(80, 32, seed=4).numpy()
    ids, gates = oracle.route(l, 4, score=W.SCORE_SIGMOID, routed_scale=2.5)
    for t in range(80):
        s = special.expit(l[t, ids[t]].astype(np.float64))
        assert np.allclose(gates[t], 2.5 * s / s.sum(), rtol=3e-7)
    assert np.allclose(gates.sum(1), 2.5, rtol=1e-6)
    ids_u, gates_u = oracle.route(l, 4, score=W.SCORE_SIGMOID, renorm=0)
    for t in range(80):
        assert np.allclose(gates_u[t], special.expit(l[t, ids_u[t]].astype(np.float64)), rtol=2e-7)


def test_hand_worked_routing_dispatch_combine():
    """Hand-worked example of the pages' definitions.

    Four tokens, four experts, top-2 softmax with renormalised gates, capacity
    factor 1.0.  Dispatch gives every token k=2 target positions and combine
    sums the k expert outputs weighted by the router weights ("Expert
    Parallelism: MoE model parallel split", §12 Q2); a per-expert capacity
    drops tokens beyond it ("Expert parallelism for MoE serving", FAQ).
    """
    ln3, ln7 = math.log(3.0), math.log(7.0)
    l = np.array([[0.0, ln3, -1.0, -2.0],      # picks e1, e0; gates 3/4, 1/4
                  [0.5, 0.5, 0.5, -1.0],       # three-way tie: e0, e1 (lower index first)
                  [-1.0, ln3, ln3, 0.0],       # tie at the top: e1, e2; gates 1/2, 1/2
                  [0.0, 0.0, -5.0, ln7]],      # e3, then the e0/e1 tie goes to e0; 7/8, 1/8
                 np.float32)
    ids, gates = oracle.route(l, 2)
    assert ids.tolist() == [[1, 0], [0, 1], [1, 2], [3, 0]]
    assert np.allclose(gates, [[0.75, 0.25], [0.5, 0.5], [0.5, 0.5], [0.875, 0.125]], rtol=1e-6)
    # A = 8 slots, C = ceil(1.0 * 8 / 4) = 2.  counts e0: 3 (t0,t1,t3), e1: 3 (t0,t1,t2),
    # e2: 1, e3: 1.  e0 keeps t0,t1 and drops t3; e1 keeps t0,t1 and drops t2.
    d = oracle.dispatch(ids, 4, capacity_factor=1.0)
    assert d["counts"].tolist() == [3, 3, 1, 1]
    assert d["offsets"].tolist() == [0, 2, 4, 5, 6]
    assert d["row_of_slot"].tolist() == [[2, 0], [1, 3], [-1, 4], [5, -1]]
    assert d["row_token"][:6].tolist() == [0, 1, 0, 1, 2, 3]
    assert d["num_dropped"] == 2
    # combine with y[r] = (r, 10 r)
    y = np.array([[r, 10 * r] for r in range(6)], np.float32)
    out = oracle.combine(y, d["row_of_slot"], gates)
    assert np.allclose(out, [[1.5, 15.0], [2.0, 20.0], [2.0, 20.0], [4.375, 43.75]], rtol=1e-6)
    # without capacity every slot is kept: k positions per token
    d2 = oracle.dispatch(ids, 4)
    assert d2["num_dropped"] == 0 and d2["offsets"].tolist() == [0, 3, 6, 7, 8]
    assert sorted(d2["row_token"].tolist()) == [0, 0, 1, 1, 2, 2, 3, 3]


def test_hand_worked_group_limited_routing():
    """E=8 experts in G=4 groups of 2, keep 2 groups, group score = best
    sigmoid (topn=1), top-3, sigmoid gates renormalised and scaled by 2.5."""
    l = np.array([[0.1, 3.0, 2.0, 2.5, -1.0, 4.0, 0.0, 0.5]], np.float32)
    # group maxima: g0 3.0, g1 2.5, g2 4.0, g3 0.5 -> keep g2, g0 -> eligible e0,e1,e4,e5
    ids, gates = oracle.route(l, 3, score=W.SCORE_SIGMOID, routed_scale=2.5, num_groups=4,
                              topk_groups=2, group_topn=1)
    assert ids.tolist() == [[5, 1, 0]]      # e3 (2.5) would win without the group limit
    s = 1 / (1 + np.exp(-np.array([4.0, 3.0, 0.1], np.float64)))
    assert np.allclose(gates[0], 2.5 * s / s.sum(), rtol=3e-7)
    # with topn=2 the group score is the sum of the two best: g0 0.525+0.953=1.478,
    # g1 0.881+0.924=1.805, g2 0.269+0.982=1.251, g3 0.5+0.622=1.122 -> keep g1, g0
    ids2, _ = oracle.route(l, 3, score=W.SCORE_SIGMOID, num_groups=4, topk_groups=2, group_topn=2)
    assert ids2.tolist() == [[1, 3, 2]]


def _kept_groups_float64(l, G, topk_groups, topn):
    E = l.shape[0]
    gs = E // G
    s = special.expit(l.astype(np.float64)).reshape(G, gs)
    sc = -np.sort(-s, axis=1)[:, :topn].sum(1)
    order = np.argsort(-sc, kind="stable")
    margin = sc[order[topk_groups - 1]] - sc[order[topk_groups]] if topk_groups < G else np.inf
    return set(order[:topk_groups].tolist()), margin


@pytest.mark.parametrize("topn", [1, 2])
def test_group_limited_routing_vs_float64_group_scores(topn):
    lay = json.load(open(os.path.join(GOLDEN, "ep8_expert_layout.json")))
    E, G = lay["num_experts"], lay["num_gpus"]
    T, k, keep = 400, 8, 4
    bias = W.log_zipf_bias(E, 1.1)
    l = W.make_logits(T, E, seed=11 + topn, bias=bias).numpy()
    ids, gates = oracle.route(l, k, score=W.SCORE_SIGMOID, routed_scale=2.5, num_groups=G,
                              topk_groups=keep, group_topn=topn)
    ranges = lay["gpu_expert_ranges"]
    checked = 0
    for t in range(T):
        kept, margin = _kept_groups_float64(l[t], G, keep, topn)
        groups_used = {g for e in ids[t] for g, (lo, hi) in enumerate(ranges) if lo <= e <= hi}
        assert len(groups_used) <= keep
        if margin > 1e-5:
            checked += 1
            assert groups_used <= kept
            eligible = np.array([e for g in sorted(kept) for e in range(ranges[g][0], ranges[g][1] + 1)])
            le = l[t, eligible]
            ref = eligible[np.argsort(-le, kind="stable")[:k]]
            assert ids[t].tolist() == ref.tolist()
        s = special.expit(l[t, ids[t]].astype(np.float64))
        assert np.allclose(gates[t], 2.5 * s / s.sum(), rtol=3e-7)
    assert checked > 0.9 * T


def test_group_limit_special_cases_reduce_to_plain_topk():
    l = W.make_logits(200, 64, seed=5, tie_fraction=0.2).numpy()
    plain, _ = oracle.route(l, 6, score=W.SCORE_SIGMOID)
    allg, _ = oracle.route(l, 6, score=W.SCORE_SIGMOID, num_groups=8, topk_groups=8, group_topn=2)
    oneg, _ = oracle.route(l, 6, score=W.SCORE_SIGMOID, num_groups=1, topk_groups=1, group_topn=2)
    assert np.array_equal(plain, allg) and np.array_equal(plain, oneg)


def test_per_token_k():
    T, E, kmax = 500, 16, 8
    l = W.make_logits(T, E, seed=9, tie_fraction=0.1).numpy()
    kpt = W.make_k_per_token(T, (1, 2, 4, 6, 8), seed=3).numpy().copy()
    kpt[::37] = 0
    kpt[5::53] = kmax + 1
    kpt[7::61] = -3
    ids, gates = oracle.route(l, kmax, k_per_token=kpt)
    for t in range(T):
        kt = kpt[t]
        if kt < 1 or kt > kmax:
            assert np.all(ids[t] == -1) and np.all(gates[t] == 0)
            continue
        assert ids[t, :kt].tolist() == stable_topk(l[t], kt).tolist()
        assert np.all(ids[t, kt:] == -1) and np.all(gates[t, kt:] == 0)
        assert abs(gates[t, :kt].sum() - 1) < 1e-6
    # k_t equal to k everywhere is the fixed-k result
    ids_f, g_f = oracle.route(l, kmax)
    ids_k, g_k = oracle.route(l, kmax, k_per_token=np.full(T, kmax, np.int32))
    assert np.array_equal(ids_f, ids_k) and np.array_equal(g_f, g_k)


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------
def library_dispatch(ids, E, C):
    """Dispatch by library routines: bincount, cumsum and a stable argsort."""
    T, k = ids.shape
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    kept = np.minimum(counts, C)
    offsets = np.concatenate([[0], np.cumsum(kept)])
    slots = np.nonzero(valid)[0]                     # token-major order
    e_of = flat[slots]
    order = np.argsort(e_of, kind="stable")         # stable: token order inside an expert
    ros = np.full(T * k, -1, np.int64)
    row_token = []
    start = np.concatenate([[0], np.cumsum(counts)])
    for e in range(E):
        grp = slots[order[start[e]:start[e + 1]]]
        keep = grp[:kept[e]]
        ros[keep] = offsets[e] + np.arange(len(keep))
        row_token.extend((keep // k).tolist())
    dropped = int(np.maximum(counts - C, 0).sum())
    return counts, offsets, ros.reshape(T, k), np.array(row_token, np.int64), dropped


@pytest.mark.parametrize("cf", [0.0, 1.25, 1.0, 0.5, 3.0])
def test_dispatch_matches_library_routines(cf):
    T, E, kmax = 700, 24, 6
    bias = W.log_zipf_bias(E, 1.2)
    l = W.make_logits(T, E, seed=21, bias=bias).numpy()
    kpt = W.make_k_per_token(T, (2, 4, 6), seed=4).numpy()
    ids, _ = oracle.route(l, kmax, k_per_token=kpt)
    d = oracle.dispatch(ids, E, capacity_factor=cf)
    A = int((ids >= 0).sum())
    C = math.ceil(cf * A / E) if cf > 0 else 10 ** 12
    counts, offsets, ros, row_token, dropped = library_dispatch(ids, E, C)
    assert np.array_equal(d["counts"], counts)
    assert np.array_equal(d["offsets"], offsets)
    assert np.array_equal(d["row_of_slot"], ros)
    R = int(offsets[-1])
    assert np.array_equal(d["row_token"][:R], row_token)
    assert d["num_dropped"] == dropped == A - R
    # bijection between kept slots and rows [0, R)
    kept_rows = d["row_of_slot"][d["row_of_slot"] >= 0]
    assert np.array_equal(np.sort(kept_rows), np.arange(R))
    # token indices strictly increase inside each expert's rows
    for e in range(E):
        seg = d["row_token"][offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_capacity_closed_forms():
    assert oracle.capacity(1.25, 81920, 128) == 800
    assert oracle.capacity(1.25, 10, 4) == 4          # ceil(3.125)
    assert oracle.capacity(1.0, 8, 4) == 2
    assert oracle.capacity(0.0, 8, 4) > 10 ** 9       # no limit
    assert oracle.capacity(-1.0, 8, 4) > 10 ** 9
    # C = 1 keeps exactly the first slot (in token order) of every expert
    l = W.make_logits(100, 10, seed=2).numpy()
    ids, _ = oracle.route(l, 3)
    d = oracle.dispatch(ids, 10, capacity_factor=1.0 / 32.0)   # ceil(300/32/10) = ceil(0.9375) = 1
    flat = ids.reshape(-1)
    for e in range(10):
        first = np.nonzero(flat == e)[0]
        if len(first):
            assert d["row_of_slot"].reshape(-1)[first[0]] == d["offsets"][e]
            assert np.all(d["row_of_slot"].reshape(-1)[first[1:]] == -1)
    # no limit equals a huge factor
    a = oracle.dispatch(ids, 10, 0.0)
    b = oracle.dispatch(ids, 10, 1e6)
    assert all(np.array_equal(a[key], b[key]) for key in ("counts", "offsets", "row_of_slot"))


# ---------------------------------------------------------------------------
# expert FFN, combine, whole layer
# ---------------------------------------------------------------------------
def dense_ffn64(X, wg, wu, wd):
    """SwiGLU FFN in float64 with library routines: silu(z) = z * expit(z)."""
    a = X @ wg.T
    u = X @ wu.T
    return (a * special.expit(a) * u) @ wd.T


@pytest.mark.parametrize("bf16", [False, True])
def test_grouped_ffn_matches_dense_float64(bf16):
    E, H, I = 4, 64, 96
    counts = [5, 0, 17, 3]
    R = sum(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    mk = (lambda s, sd: rand_bf16(s, sd, RNG)) if bf16 else \
        (lambda s, sd: (RNG.standard_normal(s) * sd).astype(np.float32))
    x = mk((R, H), 1.0)
    wg, wu = mk((E, I, H), 1 / math.sqrt(H)), mk((E, I, H), 1 / math.sqrt(H))
    wd = mk((E, H, I), 1 / math.sqrt(I))
    y = oracle.grouped_ffn(x, offsets, wg, wu, wd)
    X = widen(x).astype(np.float64)
    ref = np.zeros((R, H))
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        ref[a:b] = dense_ffn64(X[a:b], widen(wg[e]).astype(np.float64), widen(wu[e]).astype(np.float64),
                               widen(wd[e]).astype(np.float64))
    rms = np.sqrt((ref ** 2).mean())
    assert np.abs(y - ref).max() <= 1e-6 * rms
    # row subset gives the same rows
    rows = np.array([20, 0, 24, 7], np.int32)
    ys = oracle.grouped_ffn(x, offsets, wg, wu, wd, rows=rows)
    assert np.array_equal(ys, y[rows])


def test_combine_matches_sparse_matmul():
    T, E, k, H = 60, 7, 3, 33
    l = W.make_logits(T, E, seed=8).numpy()
    ids, gates = oracle.route(l, k)
    d = oracle.dispatch(ids, E, capacity_factor=0.8)
    R = d["offsets"][-1]
    y = RNG.standard_normal((R, H)).astype(np.float32)
    ys = RNG.standard_normal((T, H)).astype(np.float32)
    out = oracle.combine(y, d["row_of_slot"], gates, ys)
    S = np.zeros((T, R))
    for t in range(T):
        for j in range(k):
            r = d["row_of_slot"][t, j]
            if r >= 0:
                S[t, r] = gates[t, j]
    ref = S @ y.astype(np.float64) + ys
    assert np.abs(out - ref).max() <= 1e-6 * np.sqrt((ref ** 2).mean())


def _tiny_layer(bf16, E=6, H=64, I=80, T=48, Is=0, seed=0):
    rng = np.random.default_rng(100 + seed)
    mk = (lambda s, sd: rand_bf16(s, sd, rng)) if bf16 else \
        (lambda s, sd: (rng.standard_normal(s) * sd).astype(np.float32))
    d = dict(x=mk((T, H), 1.0), w_router=mk((E, H), 1 / math.sqrt(H)),
             w_gate=mk((E, I, H), 1 / math.sqrt(H)), w_up=mk((E, I, H), 1 / math.sqrt(H)),
             w_down=mk((E, H, I), 1 / math.sqrt(I)))
    if Is:
        d.update(ws_gate=mk((Is, H), 1 / math.sqrt(H)), ws_up=mk((Is, H), 1 / math.sqrt(H)),
                 ws_down=mk((H, Is), 1 / math.sqrt(Is)))
    return d


def _dense_masked_layer(d, gate_matrix):
    """Every expert on every token in float64, masked by the [T,E] gate matrix."""
    X = widen(d["x"]).astype(np.float64)
    out = np.zeros((X.shape[0], X.shape[1]))
    for e in range(gate_matrix.shape[1]):
        ye = dense_ffn64(X, widen(d["w_gate"][e]).astype(np.float64), widen(d["w_up"][e]).astype(np.float64),
                         widen(d["w_down"][e]).astype(np.float64))
        out += gate_matrix[:, e:e + 1] * ye
    if "ws_gate" in d:
        out += dense_ffn64(X, widen(d["ws_gate"]).astype(np.float64), widen(d["ws_up"]).astype(np.float64),
                           widen(d["ws_down"]).astype(np.float64))
    return out


@pytest.mark.parametrize("bf16,cf,Is", [(False, 0.0, 0), (True, 0.0, 0), (True, 1.0, 0), (False, 0.0, 40),
                                        (True, 0.75, 48)])
def test_layer_matches_dense_masked_evaluation(bf16, cf, Is):
    E, k = 6, 2
    d = _tiny_layer(bf16, E=E, Is=Is, seed=int(cf * 4) + Is)
    res = oracle.layer_forward(d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"], k,
                               capacity_factor=cf, ws_gate=d.get("ws_gate"), ws_up=d.get("ws_up"),
                               ws_down=d.get("ws_down"))
    # routing rebuilt from library routines on float64 logits rounded to fp32
    X = widen(d["x"]).astype(np.float64)
    l = (X @ widen(d["w_router"]).astype(np.float64).T).astype(np.float32)
    assert np.array_equal(l, res["logits"]) or np.all(np.abs(l - res["logits"]) <= np.spacing(np.abs(l)))
    T = X.shape[0]
    ids = np.stack([stable_topk(res["logits"][t], k) for t in range(T)])
    A = T * k
    C = math.ceil(cf * A / E) if cf > 0 else 10 ** 12
    _, _, ros, _, _ = library_dispatch(ids, E, C)
    G = np.zeros((T, E))
    for t in range(T):
        g = special.softmax(res["logits"][t, ids[t]].astype(np.float64))
        for j in range(k):
            if ros[t, j] >= 0:
                G[t, ids[t, j]] = g[j]
    ref = _dense_masked_layer(d, G)
    rms = np.sqrt((ref ** 2).mean())
    assert np.abs(res["out"] - ref).max() <= 2e-6 * rms
    # subset of tokens gives the same rows
    tok = np.array([5, 0, 47, 13], np.int32)
    sub = oracle.layer_forward(d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"], k,
                               capacity_factor=cf, ws_gate=d.get("ws_gate"), ws_up=d.get("ws_up"),
                               ws_down=d.get("ws_down"), tokens=tok)
    assert np.array_equal(sub["out"], res["out"][tok])


@pytest.mark.parametrize("cf", [0.0, 1.0])
def test_layer_routes_on_given_logits(cf):
    """layer_forward(logits=L) routes on L (the way a GPU's routing is
    checked given its own fp32 logits): with the oracle's own logits it is the
    default call bit for bit; with other logits the routing, dispatch and
    output follow them -- checked against the dense masked float64 layer
    built from stable argsort and library dispatch on those logits."""
    E, k = 6, 2
    d = _tiny_layer(True, E=E, seed=11)
    base = oracle.layer_forward(d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"], k, capacity_factor=cf)
    same = oracle.layer_forward(d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"], k, capacity_factor=cf,
                                logits=base["logits"])
    for key in ("out", "logits", "ids", "gates", "counts", "offsets", "row_of_slot"):
        assert np.array_equal(same[key], base[key]), key
    rng = np.random.default_rng(5)
    L = rng.standard_normal(base["logits"].shape).astype(np.float32)
    res = oracle.layer_forward(d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"], k, capacity_factor=cf,
                               logits=L)
    assert np.array_equal(res["logits"], L)
    T = L.shape[0]
    ids = np.stack([stable_topk(L[t], k) for t in range(T)])
    assert np.array_equal(res["ids"], ids)
    assert not np.array_equal(ids, base["ids"])
    C = math.ceil(cf * T * k / E) if cf > 0 else 10 ** 12
    _, _, ros, _, _ = library_dispatch(ids, E, C)
    assert np.array_equal(res["row_of_slot"], ros)
    G = np.zeros((T, E))
    for t in range(T):
        g = special.softmax(L[t, ids[t]].astype(np.float64))
        for j in range(k):
            if ros[t, j] >= 0:
                G[t, ids[t, j]] = g[j]
    ref = _dense_masked_layer(d, G)
    assert np.abs(res["out"] - ref).max() <= 2e-6 * np.sqrt((ref ** 2).mean())


def test_identical_experts_give_routing_independent_output():
    d = _tiny_layer(False, E=5, seed=3)
    for key in ("w_gate", "w_up", "w_down"):
        d[key] = np.repeat(d[key][:1], 5, axis=0)
    res = oracle.layer_forward(d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"], 3)
    X = d["x"].astype(np.float64)
    ref = dense_ffn64(X, d["w_gate"][0].astype(np.float64), d["w_up"][0].astype(np.float64),
                      d["w_down"][0].astype(np.float64))      # sum of renormalised gates = 1
    assert np.abs(res["out"] - ref).max() <= 2e-6 * np.sqrt((ref ** 2).mean())


def test_all_experts_without_renorm_is_dense_softmax_mixture():
    E = 4
    d = _tiny_layer(False, E=E, seed=4)
    res = oracle.layer_forward(d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"], E, renorm=0)
    P = special.softmax(res["logits"].astype(np.float64), axis=1)
    ref = _dense_masked_layer(d, P)
    assert np.abs(res["out"] - ref).max() <= 2e-6 * np.sqrt((ref ** 2).mean())


def test_single_expert_k1_is_dense_ffn():
    d = _tiny_layer(True, E=1, seed=5)
    res = oracle.layer_forward(d["x"], d["w_router"], d["w_gate"], d["w_up"], d["w_down"], 1)
    X = widen(d["x"]).astype(np.float64)
    ref = dense_ffn64(X, widen(d["w_gate"][0]).astype(np.float64), widen(d["w_up"][0]).astype(np.float64),
                      widen(d["w_down"][0]).astype(np.float64))
    assert np.abs(res["out"] - ref).max() <= 2e-6 * np.sqrt((ref ** 2).mean())


# ---------------------------------------------------------------------------
# workloads: the skew the synthetic bias produces
# ---------------------------------------------------------------------------
def test_deepseek_shaped_bias_reaches_hotspot_ratio():
    thr = json.load(open(os.path.join(GOLDEN, "hotspot_threshold.json")))["max_mean_threshold"]
    cfg = W.CONFIGS["deepseek_v3"].with_tokens(2048)
    import torch
    x = W.normal((cfg.tokens, cfg.hidden), 1.0, cfg.dtype, "cpu", W.seed_for(cfg.name, W.TAG_X))
    wr = W.normal((cfg.experts, cfg.hidden), 1 / math.sqrt(cfg.hidden), cfg.dtype, "cpu",
                  W.seed_for(cfg.name, W.TAG_WR))
    bias = W.log_zipf_bias(cfg.experts, cfg.zipf_s)
    l = oracle.router_logits(W.to_numpy_raw(x), W.to_numpy_raw(wr), bias)
    ids, _ = oracle.route(l, cfg.top_k, score=cfg.score, routed_scale=cfg.routed_scale,
                          num_groups=cfg.num_groups, topk_groups=cfg.topk_groups, group_topn=cfg.group_topn)
    counts = np.bincount(ids.reshape(-1), minlength=cfg.experts)
    assert counts.mean() > 0 and counts.max() / counts.mean() >= thr
    del torch


# ---- redundant experts: replica choice ------------------------------------------------------


def _rank_in_expert(ids):
    """Token-major rank of every slot among the slots of the same expert (numpy, no oracle)."""
    flat = ids.reshape(-1)
    rank = np.full(flat.shape, -1, np.int64)
    seen = {}
    for s, e in enumerate(flat.tolist()):
        if e >= 0:
            rank[s] = seen.get(e, 0)
            seen[e] = rank[s] + 1
    return rank.reshape(ids.shape)


def _random_replica_table(rng, E, max_rep):
    n = rng.integers(1, max_rep + 1, size=E)
    off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    P = int(off[-1])
    rex = rng.permutation(P).astype(np.int32)      # every physical expert holds one replica
    return off, rex, P


def test_replicas_identity_table_keeps_ids():
    rng = np.random.default_rng(7)
    ids = rng.integers(-1, 9, size=(40, 3)).astype(np.int32)
    phys, bad = oracle.map_replicas(ids, np.arange(10, dtype=np.int32), np.arange(9, dtype=np.int32), 9)
    assert bad == 0
    assert np.array_equal(phys, np.where(ids >= 0, ids, -1))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_replicas_follow_round_robin_in_token_order(seed):
    # least-loaded with ties to the lower replica index, from an empty batch, is the
    # rank-mod-n rotation: the r-th slot of e takes replica r mod n_e
    rng = np.random.default_rng(seed)
    T, E, k = 60, 6, 3
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[rng.random((T, k)) < 0.1] = -1
    off, rex, P = _random_replica_table(rng, E, 3)
    phys, bad = oracle.map_replicas(ids, off, rex, P)
    assert bad == 0
    rank = _rank_in_expert(ids)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            if e < 0:
                assert phys[t, j] == -1
                continue
            n = off[e + 1] - off[e]
            assert phys[t, j] == rex[off[e] + rank[t, j] % n]


def test_replica_loads_differ_by_at_most_one():
    rng = np.random.default_rng(11)
    T, E, k = 500, 8, 2
    logits = W.make_logits(T, E, seed=4, bias=W.log_zipf_bias(E, 1.2)).numpy()
    ids, _ = oracle.route(logits, k)
    off, rex, P = _random_replica_table(rng, E, 4)
    phys, _ = oracle.map_replicas(ids, off, rex, P)
    counts = np.bincount(ids[ids >= 0], minlength=E)
    pc = np.bincount(phys[phys >= 0], minlength=P)
    for e in range(E):
        reps = pc[rex[off[e]:off[e + 1]]]
        assert reps.sum() == counts[e]
        assert reps.max() - reps.min() <= 1
        assert np.all(np.diff(reps) <= 0)           # the extra slots go to the lower replica indices


def test_replicas_lower_the_hottest_load():
    # replicating the hottest experts of the DeepSeek-V3-shaped routing lowers max/mean
    cfg = W.CONFIGS["deepseek_v3"]
    T, E = 1024, cfg.experts
    logits = W.make_logits(T, E, seed=9, bias=W.log_zipf_bias(E, 1.1)).numpy()
    ids, _ = oracle.route(logits, cfg.top_k, None, cfg.score, cfg.renormalize, cfg.routed_scale,
                          cfg.num_groups, cfg.topk_groups, cfg.group_topn)
    counts = np.bincount(ids[ids >= 0], minlength=E)
    hot = np.argsort(-counts, kind="stable")[:16]
    n = np.ones(E, np.int64)
    n[hot] = 3                                      # two extra replicas for the 16 hottest
    off = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    rex = np.arange(off[-1], dtype=np.int32)
    phys, bad = oracle.map_replicas(ids, off, rex, int(off[-1]))
    assert bad == 0
    pc = np.bincount(phys[phys >= 0], minlength=int(off[-1]))
    assert pc.sum() == counts.sum()
    top = hot[0]
    assert pc[rex[off[top]:off[top + 1]]].max() == -(-counts[top] // 3)
    assert pc.max() / pc.mean() < counts.max() / counts.mean()


def test_replicas_invalid_table_entries():
    ids = np.array([[0, 1], [1, 2], [2, 0]], np.int32)
    off = np.array([0, 1, 1, 3], np.int32)          # expert 1 has no replica
    rex = np.array([0, 1, 7], np.int32)             # expert 2's second replica is out of range
    phys, bad = oracle.map_replicas(ids, off, rex, 3)
    assert np.array_equal(phys, [[0, -1], [-1, 1], [-1, 0]])
    assert bad == 3


def test_replicas_hand_worked():
    # expert 0 on physical 0 and 3 (in that order), experts 1 and 2 on one copy each
    ids = np.array([[0, 1], [0, 2], [0, 1], [1, 0]], np.int32)
    phys, bad = oracle.map_replicas(ids, [0, 2, 3, 4], [0, 3, 1, 2], 4)
    assert bad == 0
    assert np.array_equal(phys, [[0, 1], [3, 2], [0, 1], [1, 3]])
