"""CPU oracle for the MoE-layer forward path (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never calls it, and nothing here is a fallback
for the GPU path.  It shares no code with the GPU library: the arithmetic is in
`moe_oracle.c` (plain C, fp64 accumulation, one pass per token over its chosen
experts); this module only builds that file with gcc and marshals numpy arrays.

Activations and weights are passed as fp32 arrays or as raw bf16 bits (uint16).
Every function cites, in `moe_oracle.c`, the page passage it follows.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_SO = os.path.join(_BUILD, "libmoe_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc (no contraction, no fast math, OpenMP)."""
    if not force and os.path.exists(_SO):
        return _SO
    os.makedirs(_BUILD, exist_ok=True)
    tmp = _SO + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_SO)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.oracle_num_threads.restype = i32
        L.oracle_router_logits.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp]
        L.oracle_sigmoid_spec.argtypes = [f32]
        L.oracle_sigmoid_spec.restype = f32
        L.oracle_sigmoid_spec_array.argtypes = [ctypes.c_int64, vp, vp]
        L.oracle_route.argtypes = [i32, i32, vp, i32, vp, i32, i32, f32, i32, i32, i32, vp, vp]
        L.oracle_capacity.argtypes = [f32, ctypes.c_int64, i32]
        L.oracle_capacity.restype = ctypes.c_int64
        L.oracle_dispatch.argtypes = [i32, i32, i32, vp, f32, vp, vp, vp, vp, vp]
        L.oracle_dispatch.restype = i32
        L.oracle_map_replicas.argtypes = [i32, i32, i32, vp, vp, vp, i32, vp]
        L.oracle_map_replicas.restype = i32
        L.oracle_grouped_ffn.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp]
        L.oracle_combine.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_e4m3_value.argtypes = [i32]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_mxfp8_quantize.argtypes = [i32, i32, i32, vp, vp, vp]
        L.oracle_grouped_ffn_mxfp8.argtypes = [i32, i32, i32] + [vp] * 9 + [vp, i32, vp, vp]
        L.oracle_ep_layout.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.oracle_ep_layout.restype = i32
        L.oracle_ep_combine.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.oracle_layer_forward.argtypes = (
            [i32] * 6 + [vp, vp, vp, vp] + [i32, i32, f32, i32, i32, i32, f32] + [vp, vp, vp]
            + [i32, vp, vp, vp] + [vp, i32, vp] + [vp] * 8 + [vp])
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _act(a: np.ndarray):
    """(contiguous array, dtype code) for fp32 or raw-bf16 input."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return a, 1
    if a.dtype != np.float32:
        raise TypeError(f"oracle expects float32 or raw bf16 (uint16), got {a.dtype}")
    return a, 0


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def router_logits(x, w_router, bias=None) -> np.ndarray:
    x, dt = _act(x)
    w, dt2 = _act(w_router)
    assert dt == dt2
    T, H = x.shape
    E = w.shape[0]
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((T, E), np.float32)
    lib().oracle_router_logits(T, H, E, dt, _p(x), _p(w), _p(b), _p(out))
    return out


def sigmoid_spec(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    lib().oracle_sigmoid_spec_array(x.size, _p(x), _p(y))
    return y


def route(logits, k_max, k_per_token=None, score=0, renorm=1, routed_scale=1.0, num_groups=1,
          topk_groups=1, group_topn=0):
    l = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = l.shape
    kpt = None if k_per_token is None else np.ascontiguousarray(k_per_token, dtype=np.int32)
    ids = np.empty((T, k_max), np.int32)
    gates = np.empty((T, k_max), np.float32)
    lib().oracle_route(T, E, _p(l), k_max, _p(kpt), score, renorm, routed_scale, num_groups,
                       topk_groups, group_topn, _p(ids), _p(gates))
    return ids, gates


def capacity(cf: float, A: int, E: int) -> int:
    return int(lib().oracle_capacity(cf, A, E))


def dispatch(ids, E, capacity_factor=0.0):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    ros = np.empty((T, k), np.int32)
    row_token = np.full(T * k, -1, np.int32)
    nd = np.zeros(1, np.int32)
    R = lib().oracle_dispatch(T, E, k, _p(ids), capacity_factor, _p(counts), _p(offsets), _p(ros),
                              _p(row_token), _p(nd))
    return dict(counts=counts, offsets=offsets, row_of_slot=ros, row_token=row_token,
                num_dropped=int(nd[0]), R=int(R))


def map_replicas(ids, replica_offsets, replica_experts, num_physical):
    """Physical expert of every slot (least-loaded replica, token-major order)
    and the number of slots whose replica-table entry was invalid."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    E = len(replica_offsets) - 1
    ro = np.ascontiguousarray(replica_offsets, dtype=np.int32)
    rex = np.ascontiguousarray(replica_experts, dtype=np.int32)
    if rex.size == 0:
        rex = np.zeros(1, np.int32)
    phys = np.empty((T, k), np.int32)
    bad = lib().oracle_map_replicas(T, E, k, _p(ids), _p(ro), _p(rex), int(num_physical), _p(phys))
    return phys, int(bad)


def ep_layout(ids, gates, E, G):
    """Send layout of the dispatch exchange over G ranks (experts in G
    contiguous blocks): one row per (rank, token) pair with any of the
    token's experts on that rank, destination-major, tokens ascending.
    Returns dict(rank_counts, rank_offsets, send_token, send_ids (local expert
    ids), send_gates, slot_send_pos, S = rows sent)."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    g = np.ascontiguousarray(gates, dtype=np.float32)
    T, k = ids.shape
    n_rows = T * min(k, G)
    rc = np.empty(G, np.int32)
    ro = np.empty(G + 1, np.int32)
    st = np.empty(n_rows, np.int32)
    sid = np.empty((n_rows, k), np.int32)
    sg = np.empty((n_rows, k), np.float32)
    ssp = np.empty((T, k), np.int32)
    S = lib().oracle_ep_layout(T, E, k, G, _p(ids), _p(g), _p(rc), _p(ro), _p(st), _p(sid), _p(sg), _p(ssp))
    return dict(rank_counts=rc, rank_offsets=ro, send_token=st, send_ids=sid, send_gates=sg, slot_send_pos=ssp,
                S=int(S))


def ep_combine(partial, slot_send_pos, y_shared=None) -> np.ndarray:
    """out[t] = sum over the token's distinct send rows (ascending) of
    partial[row] (+ y_shared[t])."""
    pt = np.ascontiguousarray(partial, dtype=np.float32)
    ssp = np.ascontiguousarray(slot_send_pos, dtype=np.int32)
    T, k = ssp.shape
    H = pt.shape[1]
    ys = None if y_shared is None else np.ascontiguousarray(y_shared, dtype=np.float32)
    out = np.empty((T, H), np.float32)
    lib().oracle_ep_combine(T, H, k, _p(pt), _p(ssp), _p(ys), _p(out))
    return out


def grouped_ffn(x_perm, offsets, w_gate, w_up, w_down, rows=None) -> np.ndarray:
    x, dt = _act(x_perm)
    wg, _ = _act(w_gate)
    wu, _ = _act(w_up)
    wd, _ = _act(w_down)
    E, I, H = wg.shape
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    n = int(off[E]) if r is None else len(r)
    y = np.empty((n, H), np.float32)
    lib().oracle_grouped_ffn(E, H, I, dt, _p(x), _p(off), _p(wg), _p(wu), _p(wd), _p(r),
                             0 if r is None else len(r), _p(y))
    return y


def combine(y_perm, row_of_slot, gates, y_shared=None) -> np.ndarray:
    y = np.ascontiguousarray(y_perm, dtype=np.float32)
    ros = np.ascontiguousarray(row_of_slot, dtype=np.int32)
    g = np.ascontiguousarray(gates, dtype=np.float32)
    ys = None if y_shared is None else np.ascontiguousarray(y_shared, dtype=np.float32)
    T, k = ros.shape
    H = y.shape[1]
    out = np.empty((T, H), np.float32)
    lib().oracle_combine(T, H, k, _p(y), _p(ros), _p(g), _p(ys), _p(out))
    return out


def layer_forward(x, w_router, w_gate, w_up, w_down, k_max, bias=None, k_per_token=None,
                  score=0, renorm=1, routed_scale=1.0, num_groups=1, topk_groups=1, group_topn=0,
                  capacity_factor=0.0, ws_gate=None, ws_up=None, ws_down=None, tokens=None, logits=None):
    """Whole layer; returns dict(out=[n,H] for `tokens` (or all), plus routing).
    logits (optional, [T,E] fp32): route on these instead of the oracle's own
    router logits (for comparing routing given the same fp32 logits)."""
    x, dt = _act(x)
    wr, _ = _act(w_router)
    wg, _ = _act(w_gate)
    wu, _ = _act(w_up)
    wd, _ = _act(w_down)
    T, H = x.shape
    E, I, _ = wg.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    kpt = None if k_per_token is None else np.ascontiguousarray(k_per_token, dtype=np.int32)
    if ws_gate is not None:
        sg, _ = _act(ws_gate)
        su, _ = _act(ws_up)
        sd, _ = _act(ws_down)
        Is = sg.shape[0]
    else:
        sg = su = sd = None
        Is = 0
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n = T if tok is None else len(tok)
    out = np.empty((n, H), np.float32)
    ids = np.empty((T, k_max), np.int32)
    gates = np.empty((T, k_max), np.float32)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    ros = np.empty((T, k_max), np.int32)
    row_token = np.full(T * k_max, -1, np.int32)
    nd = np.zeros(1, np.int32)
    lin = None
    if logits is not None:
        lin = np.ascontiguousarray(logits, dtype=np.float32)
        assert lin.shape == (T, E), lin.shape
    logits = np.empty((T, E), np.float32)
    lib().oracle_layer_forward(T, H, E, I, k_max, dt, _p(x), _p(wr), _p(b), _p(kpt), score, renorm,
                               routed_scale, num_groups, topk_groups, group_topn, capacity_factor,
                               _p(wg), _p(wu), _p(wd), Is, _p(sg), _p(su), _p(sd), _p(tok),
                               0 if tok is None else len(tok), _p(out), _p(logits), _p(ids),
                               _p(gates), _p(counts), _p(offsets), _p(ros), _p(row_token), _p(nd),
                               _p(lin))
    return dict(out=out, logits=logits, ids=ids, gates=gates, counts=counts, offsets=offsets,
                row_of_slot=ros, row_token=row_token, num_dropped=int(nd[0]))


def layer_forward_cfg(cfg, inputs_np, tokens=None, logits=None):
    """layer_forward with the routing options of a workloads.LayerConfig."""
    i = inputs_np
    return layer_forward(i["x"], i["w_router"], i["w_gate"], i["w_up"], i["w_down"], cfg.top_k,
                         bias=i.get("bias"), k_per_token=i.get("k_per_token"), score=cfg.score,
                         renorm=cfg.renormalize, routed_scale=cfg.routed_scale,
                         num_groups=cfg.num_groups, topk_groups=cfg.topk_groups,
                         group_topn=cfg.group_topn, capacity_factor=cfg.capacity_factor,
                         ws_gate=i.get("ws_gate"), ws_up=i.get("ws_up"), ws_down=i.get("ws_down"),
                         tokens=tokens, logits=logits)


# ---- MXFP8 (OCP Microscaling MXFP8, E4M3 elements, 32-element blocks) --------

def e4m3_value(codes) -> np.ndarray:
    """Value of each E4M3 code (float64; NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.int64)
    L = lib()
    table = np.array([L.oracle_e4m3_value(i) for i in range(256)], np.float64)
    return table[c]


def mxfp8_quantize(a):
    """MXFP8 quantisation along the last axis: (codes uint8 [..., K],
    scales uint8 [..., K/32]); a is float32 or raw bf16 (uint16)."""
    a, dt = _act(a)
    K = a.shape[-1]
    if K % 32:
        raise ValueError("the last axis must be a multiple of 32")
    rows = a.size // K
    codes = np.empty(a.shape, np.uint8)
    scales = np.empty(a.shape[:-1] + (K // 32,), np.uint8)
    lib().oracle_mxfp8_quantize(rows, K, dt, _p(a), _p(codes), _p(scales))
    return codes, scales


def mxfp8_decode(codes, scales) -> np.ndarray:
    """code * 2^(scale - 127), float64 (exact)."""
    v = e4m3_value(codes)
    sc = np.repeat(np.asarray(scales, dtype=np.int64), 32, axis=-1)
    return np.ldexp(v, sc - 127)


def grouped_ffn_mxfp8(xq, xs, offsets, w_gate, w_up, w_down, rows=None, return_h=False):
    """Grouped SwiGLU FFN on MXFP8 permuted rows; each weight is a
    (codes, scales) pair from mxfp8_quantize ([E,I,H] gate/up, [E,H,I] down).
    Returns y [n,H] fp32, or (y, h) with h [n,I] the fp32 SwiGLU activations
    before their MXFP8 rounding when return_h."""
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    xs = np.ascontiguousarray(xs, dtype=np.uint8)
    (gq, gs), (uq, us), (dq, ds) = [(np.ascontiguousarray(c, dtype=np.uint8),
                                     np.ascontiguousarray(sc, dtype=np.uint8))
                                    for c, sc in (w_gate, w_up, w_down)]
    E, I, H = gq.shape
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    n = int(off[E]) if r is None else len(r)
    y = np.empty((n, H), np.float32)
    h = np.empty((n, I), np.float32) if return_h else None
    lib().oracle_grouped_ffn_mxfp8(E, H, I, _p(xq), _p(xs), _p(off), _p(gq), _p(gs), _p(uq), _p(us),
                                   _p(dq), _p(ds), _p(r), 0 if r is None else len(r), _p(y), _p(h))
    return (y, h) if return_h else y


def layer_forward_mxfp8(x, w_router, wq, k_max, bias=None, k_per_token=None, score=0, renorm=1,
                        routed_scale=1.0, num_groups=1, topk_groups=1, group_topn=0,
                        capacity_factor=0.0, shared=None, tokens=None, logits=None):
    """Layer with MXFP8 experts: routing on the high-precision x and router
    (as layer_forward), x quantised to MXFP8 per token, the kept rows through
    grouped_ffn_mxfp8, the weighted sum as combine.  wq / shared: dicts with
    (codes, scales) pairs under "gate", "up", "down".  Returns dict(out=[n,H]
    for `tokens` (or all tokens), the routing, and the FFN rows computed:
    need (kept rows, ascending), ros_c (row_of_slot of `tokens` as indices
    into need), h / h_shared (fp32 SwiGLU activations before their MXFP8
    rounding, per need row / per token)).  logits (optional, [T,E] fp32): route on
    these instead of the oracle's own router logits."""
    if logits is None:
        logits = router_logits(x, w_router, bias)
    else:
        logits = np.ascontiguousarray(logits, dtype=np.float32)
    ids, gates = route(logits, k_max, k_per_token, score, renorm, routed_scale, num_groups,
                       topk_groups, group_topn)
    E = wq["gate"][0].shape[0]
    d = dispatch(ids, E, capacity_factor)
    xq, xs = mxfp8_quantize(x)
    T, H = xq.shape
    tok = np.arange(T, dtype=np.int32) if tokens is None else np.asarray(tokens, dtype=np.int32)
    ros = d["row_of_slot"][tok]
    need = np.unique(ros[ros >= 0]).astype(np.int32)
    rt = d["row_token"][:d["R"]]
    y, h = grouped_ffn_mxfp8(xq[rt], xs[rt], d["offsets"], wq["gate"], wq["up"], wq["down"], rows=need,
                             return_h=True)
    ros_c = np.where(ros >= 0, np.searchsorted(need, np.maximum(ros, 0)), -1).astype(np.int32)
    y_sh = h_sh = None
    if shared is not None:
        y_sh, h_sh = grouped_ffn_mxfp8(xq[tok], xs[tok], np.array([0, len(tok)], np.int32),
                                       *[tuple(a[None] for a in shared[n]) for n in ("gate", "up", "down")],
                                       return_h=True)
    out = combine(y if len(need) else np.zeros((1, H), np.float32), ros_c, gates[tok], y_sh)
    return dict(out=out, logits=logits, ids=ids, gates=gates, xq=xq, xs=xs, need=need, ros_c=ros_c, h=h,
                h_shared=h_sh, **d)
