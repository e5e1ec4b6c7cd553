"""ctypes binding of libmoe_mi355x.so: the C-ABI entry points under the same names.

Argument marshalling only: tensors are passed as their device pointers, the
stream as the current torch stream's hipStream_t.  Every step of the layer runs
in the library's HIP kernels; there is no other implementation behind these
functions, and a missing library raises instead of falling back.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_F16 = 0, 1, 2
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_FLAG_BAD_K, MOE_FLAG_BAD_EXPERT, MOE_FLAG_H_RANGE, MOE_FLAG_BAD_REPLICA, MOE_FLAG_Y_RANGE = 1, 2, 4, 8, 16

EXPORTED = ("moe_workspace_size", "moe_route_topk", "moe_dispatch", "moe_map_replicas", "moe_grouped_ffn",
            "moe_combine", "moe_layer_forward", "moe_group_score_sigmoid", "moe_status_string",
            "moe_last_hip_error", "moe_read_device_flags", "moe_quantize_mxfp8", "moe_workspace_size_mxfp8",
            "moe_grouped_ffn_mxfp8", "moe_layer_forward_mxfp8", "moe_layer_forward_noalloc",
            "moe_ep_dispatch_layout", "moe_ep_combine", "moe_convert_bf16_to_f16")
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20


class MoeShape(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("score", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("routed_scale", ctypes.c_float),
                ("num_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
                ("group_topn", ctypes.c_int32), ("capacity_factor", ctypes.c_float),
                ("shared_intermediate", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("down_dtype", ctypes.c_int32)]


MOE_STAGES = ("router", "route", "dispatch", "gather", "gate_up", "down", "shared", "combine")


class MoeDebug(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p),
                ("topk_gates", ctypes.c_void_p), ("expert_counts", ctypes.c_void_p),
                ("expert_offsets", ctypes.c_void_p), ("row_of_slot", ctypes.c_void_p),
                ("num_dropped", ctypes.c_void_p),
                ("stage_start", ctypes.c_void_p * len(MOE_STAGES)),
                ("stage_stop", ctypes.c_void_p * len(MOE_STAGES)),
                ("row_token", ctypes.c_void_p)]


class MoeMxfp8Ffn(ctypes.Structure):
    """moe_mxfp8_ffn: E4M3 codes and MX scales of the gate, up and down weights."""
    _fields_ = [("gate", ctypes.c_void_p), ("gate_scales", ctypes.c_void_p),
                ("up", ctypes.c_void_p), ("up_scales", ctypes.c_void_p),
                ("down", ctypes.c_void_p), ("down_scales", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().moe_status_string(status).decode()
        if status == MOE_ERR_HIP:
            msg += f" (hipError {lib().moe_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"HIP library not built: {LIB_PATH} (run python -m expert_serving_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, st, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        sp = ctypes.POINTER(MoeShape)
        L.moe_workspace_size.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_route_topk.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_dispatch.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_map_replicas.argtypes = [sp, vp, vp, vp, ctypes.c_int32, vp, vp, sz, vp]
        L.moe_grouped_ffn.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_combine.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        L.moe_layer_forward.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        ctypes.POINTER(MoeDebug), vp, sz, vp]
        L.moe_layer_forward_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                ctypes.POINTER(MoeDebug), vp]
        L.moe_ep_dispatch_layout.argtypes = [sp, ctypes.c_int32] + [vp] * 11 + [sz, vp]
        L.moe_ep_combine.argtypes = [sp, ctypes.c_int32, vp, vp, vp, vp, vp]
        L.moe_group_score_sigmoid.argtypes = [vp, vp, ctypes.c_int64, vp]
        L.moe_status_string.argtypes = [st]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_hip_error.restype = ctypes.c_int32
        L.moe_read_device_flags.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32)]
        i32, mp = ctypes.c_int32, ctypes.POINTER(MoeMxfp8Ffn)
        L.moe_quantize_mxfp8.argtypes = [i32, i32, i32, vp, i32, vp, vp, vp]
        L.moe_convert_bf16_to_f16.argtypes = [ctypes.c_int64, vp, vp, vp]
        L.moe_workspace_size_mxfp8.argtypes = [sp, ctypes.POINTER(ctypes.c_size_t)]
        L.moe_grouped_ffn_mxfp8.argtypes = [sp, vp, vp, i32, vp, mp, vp, vp, sz, vp]
        L.moe_layer_forward_mxfp8.argtypes = [sp, vp, vp, vp, vp, mp, mp, vp, ctypes.POINTER(MoeDebug), vp,
                                              sz, vp]
        for name in EXPORTED:
            if name not in ("moe_status_string", "moe_last_hip_error"):
                getattr(L, name).restype = st
        _lib = L
    return _lib


def make_shape(cfg=None, **kw) -> MoeShape:
    """A moe_shape from a workloads.LayerConfig and/or keyword overrides."""
    d = dict(num_tokens=0, hidden=0, num_experts=0, intermediate=0, top_k=1, score=0, renormalize=1,
             routed_scale=1.0, num_groups=1, topk_groups=1, group_topn=0, capacity_factor=0.0,
             shared_intermediate=0, act_dtype=MOE_BF16, out_dtype=MOE_F32, down_dtype=0)
    if cfg is not None:
        d.update(num_tokens=cfg.tokens, hidden=cfg.hidden, num_experts=cfg.experts,
                 intermediate=cfg.inter, top_k=cfg.top_k, score=cfg.score, renormalize=cfg.renormalize,
                 routed_scale=cfg.routed_scale, num_groups=cfg.num_groups, topk_groups=cfg.topk_groups,
                 group_topn=cfg.group_topn, capacity_factor=cfg.capacity_factor,
                 shared_intermediate=cfg.shared_inter, act_dtype=cfg.dtype)
    d.update(kw)
    return MoeShape(**d)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def moe_workspace_size(shape: MoeShape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(shape), ctypes.byref(n)), "moe_workspace_size")
    return int(n.value)


def moe_route_topk(shape, x, w_router, router_bias, logits_in, logits_out, k_per_token, topk_ids,
                   topk_gates, ws, ws_bytes=None, stream=None):
    _check(lib().moe_route_topk(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias),
                                _ptr(logits_in), _ptr(logits_out), _ptr(k_per_token), _ptr(topk_ids),
                                _ptr(topk_gates), _ptr(ws), ws.numel() if ws_bytes is None else ws_bytes,
                                _stream(stream)), "moe_route_topk")


def moe_dispatch(shape, x, topk_ids, expert_counts, expert_offsets, row_of_slot, row_token, num_dropped,
                 x_perm, ws, ws_bytes=None, stream=None):
    _check(lib().moe_dispatch(ctypes.byref(shape), _ptr(x), _ptr(topk_ids), _ptr(expert_counts),
                              _ptr(expert_offsets), _ptr(row_of_slot), _ptr(row_token), _ptr(num_dropped),
                              _ptr(x_perm), _ptr(ws), ws.numel() if ws_bytes is None else ws_bytes,
                              _stream(stream)), "moe_dispatch")


def moe_map_replicas(shape, topk_ids, replica_offsets, replica_experts, num_physical, phys_ids, ws,
                     ws_bytes=None, stream=None):
    _check(lib().moe_map_replicas(ctypes.byref(shape), _ptr(topk_ids), _ptr(replica_offsets),
                                  _ptr(replica_experts), int(num_physical), _ptr(phys_ids), _ptr(ws),
                                  ws.numel() if ws_bytes is None else ws_bytes, _stream(stream)),
           "moe_map_replicas")


def moe_grouped_ffn(shape, x_perm, expert_offsets, w_gate, w_up, w_down, y_perm, ws, ws_bytes=None,
                    stream=None):
    _check(lib().moe_grouped_ffn(ctypes.byref(shape), _ptr(x_perm), _ptr(expert_offsets), _ptr(w_gate),
                                 _ptr(w_up), _ptr(w_down), _ptr(y_perm), _ptr(ws),
                                 ws.numel() if ws_bytes is None else ws_bytes, _stream(stream)),
           "moe_grouped_ffn")


def moe_combine(shape, y_perm, row_of_slot, topk_gates, y_shared, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(shape), _ptr(y_perm), _ptr(row_of_slot), _ptr(topk_gates),
                             _ptr(y_shared), _ptr(out), _stream(stream)), "moe_combine")


def moe_layer_forward(shape, x, w_router, router_bias, k_per_token, w_gate, w_up, w_down, ws_gate, ws_up,
                      ws_down, out, dbg: Optional[dict], ws, ws_bytes=None, stream=None):
    d = None
    if isinstance(dbg, MoeDebug):
        d = dbg
    elif dbg:
        d = MoeDebug(**{k: _ptr(v) for k, v in dbg.items()})
    _check(lib().moe_layer_forward(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias),
                                   _ptr(k_per_token), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                   _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(out),
                                   ctypes.byref(d) if d is not None else None, _ptr(ws),
                                   ws.numel() if ws_bytes is None else ws_bytes, _stream(stream)),
           "moe_layer_forward")


def moe_layer_forward_noalloc(shape, x, w_router, router_bias, k_per_token, w_gate, w_up, w_down, ws_gate,
                              ws_up, ws_down, out, dbg: Optional[dict], stream=None):
    d = None
    if isinstance(dbg, MoeDebug):
        d = dbg
    elif dbg:
        d = MoeDebug(**{k: _ptr(v) for k, v in dbg.items()})
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias),
                                           _ptr(k_per_token), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                           _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down), _ptr(out),
                                           ctypes.byref(d) if d is not None else None, _stream(stream)),
           "moe_layer_forward_noalloc")


def moe_ep_dispatch_layout(shape, num_ranks, topk_ids, topk_gates, x, rank_counts, rank_offsets, send_token,
                           send_ids, send_gates, slot_send_pos, send_x, ws, ws_bytes=None, stream=None):
    _check(lib().moe_ep_dispatch_layout(ctypes.byref(shape), int(num_ranks), _ptr(topk_ids), _ptr(topk_gates),
                                        _ptr(x), _ptr(rank_counts), _ptr(rank_offsets), _ptr(send_token),
                                        _ptr(send_ids), _ptr(send_gates), _ptr(slot_send_pos), _ptr(send_x),
                                        _ptr(ws), ws.numel() if ws_bytes is None else ws_bytes, _stream(stream)),
           "moe_ep_dispatch_layout")


def moe_ep_combine(shape, num_ranks, partial, slot_send_pos, y_shared, out, stream=None):
    _check(lib().moe_ep_combine(ctypes.byref(shape), int(num_ranks), _ptr(partial), _ptr(slot_send_pos),
                                _ptr(y_shared), _ptr(out), _stream(stream)), "moe_ep_combine")


def moe_group_score_sigmoid(x, y, n=None, stream=None):
    _check(lib().moe_group_score_sigmoid(_ptr(x), _ptr(y), x.numel() if n is None else n, _stream(stream)),
           "moe_group_score_sigmoid")


def moe_read_device_flags(ws, stream=None) -> int:
    f = ctypes.c_uint32(0)
    _check(lib().moe_read_device_flags(_ptr(ws), _stream(stream), ctypes.byref(f)), "moe_read_device_flags")
    return int(f.value)


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_last_hip_error() -> int:
    return int(lib().moe_last_hip_error())


# ---- MXFP8 experts -----------------------------------------------------------

def moe_quantize_mxfp8(rows, cols, src_dtype, src, scale_stride, codes, scales, stream=None):
    _check(lib().moe_quantize_mxfp8(int(rows), int(cols), int(src_dtype), _ptr(src), int(scale_stride),
                                    _ptr(codes), _ptr(scales), _stream(stream)), "moe_quantize_mxfp8")


def moe_convert_bf16_to_f16(n, src, dst, stream=None):
    _check(lib().moe_convert_bf16_to_f16(int(n), _ptr(src), _ptr(dst), _stream(stream)), "moe_convert_bf16_to_f16")


def to_f16_weights(w, stream=None):
    """fp16 copy (a float16 tensor) of a bf16 device weight tensor, made by the
    library's conversion, for shapes with down_dtype = MOE_F16."""
    import torch
    assert w.dtype == torch.bfloat16
    out = torch.empty(w.shape, dtype=torch.float16, device=w.device)
    moe_convert_bf16_to_f16(w.numel(), w.contiguous(), out, stream)
    return out


def mx_scale_bytes(rows: int, cols: int, stride: Optional[int] = None) -> int:
    """Bytes of the MX scales of a [rows][cols] matrix with the given stride."""
    return (cols // 128) * (rows if stride is None else stride) * 4


def quantize_mxfp8(t, scale_stride: Optional[int] = None, stream=None):
    """(codes uint8 [..., K], scales uint8) of a bf16 / fp32 device tensor whose
    leading dimensions are flattened into rows; the codes keep t's shape."""
    import torch
    K = t.shape[-1]
    rows = t.numel() // K
    stride = rows if scale_stride is None else scale_stride
    codes = torch.empty(t.shape, dtype=torch.uint8, device=t.device)
    scales = torch.empty(max(mx_scale_bytes(rows, K, stride), 16), dtype=torch.uint8, device=t.device)
    dt = MOE_BF16 if t.dtype == torch.bfloat16 else MOE_F32
    moe_quantize_mxfp8(rows, K, dt, t.contiguous(), stride, codes, scales, stream)
    return codes, scales


def mxfp8_ffn(gate, up, down, stream=None):
    """Quantised weights of one FFN (routed [E][I][H] / [E][H][I], or shared
    [Is][H] / [H][Is]): dict of the device tensors plus the struct under "abi"."""
    g = quantize_mxfp8(gate, stream=stream)
    u = quantize_mxfp8(up, stream=stream)
    d = quantize_mxfp8(down, stream=stream)
    st = MoeMxfp8Ffn(_ptr(g[0]), _ptr(g[1]), _ptr(u[0]), _ptr(u[1]), _ptr(d[0]), _ptr(d[1]))
    return dict(gate=g, up=u, down=d, abi=st)


def _mx(w):
    if w is None:
        return None
    return ctypes.byref(w["abi"] if isinstance(w, dict) else w)


def moe_workspace_size_mxfp8(shape: MoeShape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size_mxfp8(ctypes.byref(shape), ctypes.byref(n)), "moe_workspace_size_mxfp8")
    return int(n.value)


def moe_grouped_ffn_mxfp8(shape, x_codes, x_scales, x_scale_stride, expert_offsets, experts, y_perm, ws,
                          ws_bytes=None, stream=None):
    _check(lib().moe_grouped_ffn_mxfp8(ctypes.byref(shape), _ptr(x_codes), _ptr(x_scales), int(x_scale_stride),
                                       _ptr(expert_offsets), _mx(experts), _ptr(y_perm), _ptr(ws),
                                       ws.numel() if ws_bytes is None else ws_bytes, _stream(stream)),
           "moe_grouped_ffn_mxfp8")


def moe_layer_forward_mxfp8(shape, x, w_router, router_bias, k_per_token, experts, shared, out,
                            dbg: Optional[dict], ws, ws_bytes=None, stream=None):
    d = None
    if isinstance(dbg, MoeDebug):
        d = dbg
    elif dbg:
        d = MoeDebug(**{k: _ptr(v) for k, v in dbg.items()})
    _check(lib().moe_layer_forward_mxfp8(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(router_bias),
                                         _ptr(k_per_token), _mx(experts), _mx(shared), _ptr(out),
                                         ctypes.byref(d) if d is not None else None, _ptr(ws),
                                         ws.numel() if ws_bytes is None else ws_bytes, _stream(stream)),
           "moe_layer_forward_mxfp8")
