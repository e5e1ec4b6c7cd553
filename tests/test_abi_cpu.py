"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects bad arguments on the host before enqueuing anything.

No test here launches a kernel: every call either fails validation or has
num_tokens == 0, and the pointers passed are never dereferenced.
"""

import ctypes
import os
import re

import pytest

from expert_serving_amd import abi
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")
FAKE = 0x10000          # aligned, never dereferenced
FAKE_ODD = 0x10004      # 4-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*|int32_t)\s+(moe_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    L = abi.lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(abi.EXPORTED)


def test_status_strings():
    for s in (0, -1, -2, -3, -4):
        assert abi.moe_status_string(s)
    assert abi.moe_last_hip_error() == 0


def base_shape(**kw):
    return abi.make_shape(W.CONFIGS["mixtral_prefill"], **kw)


@pytest.mark.parametrize("bad,status", [
    (dict(num_tokens=-1), abi.MOE_ERR_INVALID_ARG),
    (dict(hidden=0), abi.MOE_ERR_INVALID_ARG),
    (dict(num_experts=0), abi.MOE_ERR_INVALID_ARG),
    (dict(num_experts=513, top_k=2), abi.MOE_ERR_UNSUPPORTED),
    (dict(top_k=0), abi.MOE_ERR_INVALID_ARG),
    (dict(top_k=9), abi.MOE_ERR_INVALID_ARG),              # k > E
    (dict(num_experts=64, top_k=17), abi.MOE_ERR_UNSUPPORTED),
    (dict(score=2), abi.MOE_ERR_INVALID_ARG),
    (dict(renormalize=2), abi.MOE_ERR_INVALID_ARG),
    (dict(routed_scale=float("nan")), abi.MOE_ERR_INVALID_ARG),
    (dict(capacity_factor=float("inf")), abi.MOE_ERR_INVALID_ARG),
    (dict(act_dtype=7), abi.MOE_ERR_INVALID_ARG),
    (dict(out_dtype=7), abi.MOE_ERR_INVALID_ARG),
    (dict(hidden=4000), abi.MOE_ERR_UNSUPPORTED),           # bf16 needs multiples of 64
    (dict(intermediate=100), abi.MOE_ERR_UNSUPPORTED),
    (dict(shared_intermediate=-1), abi.MOE_ERR_INVALID_ARG),
    (dict(shared_intermediate=96), abi.MOE_ERR_UNSUPPORTED),
    (dict(num_groups=3), abi.MOE_ERR_INVALID_ARG),          # 8 % 3 != 0
    (dict(num_groups=4, topk_groups=0), abi.MOE_ERR_INVALID_ARG),
    (dict(num_groups=4, topk_groups=5), abi.MOE_ERR_INVALID_ARG),
    (dict(num_groups=4, topk_groups=1, group_topn=3), abi.MOE_ERR_INVALID_ARG),  # > E/G
    (dict(num_groups=8, topk_groups=1, top_k=2), abi.MOE_ERR_INVALID_ARG),      # 1 group of 1 < k
    (dict(act_dtype=abi.MOE_F32, hidden=4098), abi.MOE_ERR_UNSUPPORTED),
    (dict(down_dtype=5), abi.MOE_ERR_INVALID_ARG),
    (dict(down_dtype=abi.MOE_F16, act_dtype=abi.MOE_F32), abi.MOE_ERR_UNSUPPORTED),
    # int32 element offsets: T*H, I*H and E*H must stay below 2^31
    (dict(num_tokens=524288, hidden=4096), abi.MOE_ERR_UNSUPPORTED),
    (dict(num_tokens=16, intermediate=524288, hidden=4096), abi.MOE_ERR_UNSUPPORTED),
    (dict(num_tokens=16, num_experts=512, top_k=2, hidden=4194304), abi.MOE_ERR_UNSUPPORTED),
    (dict(num_tokens=16, shared_intermediate=524288, hidden=4096), abi.MOE_ERR_UNSUPPORTED),
])
def test_shape_validation(bad, status):
    s = base_shape(**bad)
    n = ctypes.c_size_t(0)
    assert abi.lib().moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == status


def test_workspace_size_grows_with_tokens():
    a = abi.moe_workspace_size(base_shape(num_tokens=64))
    b = abi.moe_workspace_size(base_shape(num_tokens=4096))
    assert 0 < a < b
    # h and y of T*k rows dominate (the gather is fused, x_perm is not kept)
    s = W.CONFIGS["mixtral_prefill"]
    assert b >= s.tokens * s.top_k * (s.inter * 2 + s.hidden * 4)


def test_workspace_holds_down_projection_parts():
    """A Mixtral-shaped layer of 256 or 512 tokens has at most 64 down tiles of
    256 rows at an even load, so its down projection splits K = 14336 in
    three and y holds three partial sums; at 1024 tokens and more, one."""
    for T, parts in ((256, 3), (512, 3), (1024, 1), (4096, 1)):
        c = W.CONFIGS["mixtral_prefill"].with_tokens(T)
        slots = T * c.top_k
        ws = abi.moe_workspace_size(abi.make_shape(c))
        assert slots * (2 * c.inter + parts * 4 * c.hidden) <= ws < slots * (2 * c.inter + (parts + 1) * 4 * c.hidden)


def test_null_and_misaligned_pointers_rejected_before_launch():
    L = abi.lib()
    s = base_shape(num_tokens=16)
    ws = abi.moe_workspace_size(s)
    ref = ctypes.byref(s)
    # route: missing outputs, misaligned x, no workspace
    assert L.moe_route_topk(ref, FAKE, FAKE, None, None, None, None, None, FAKE, FAKE, ws, None) == -1
    assert L.moe_route_topk(ref, FAKE_ODD, FAKE, None, None, None, None, FAKE, FAKE, FAKE, ws, None) == -1
    assert L.moe_route_topk(ref, FAKE, FAKE, None, None, None, None, FAKE, FAKE, None, ws, None) == -1
    assert L.moe_route_topk(ref, FAKE, FAKE, None, None, None, None, FAKE, FAKE, FAKE, ws - 1, None) == -3
    # dispatch: x without x_perm
    assert L.moe_dispatch(ref, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, ws, None) == -1
    assert L.moe_dispatch(ref, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, ws // 2, None) == -3
    # grouped ffn / combine / layer: missing weights or output
    assert L.moe_grouped_ffn(ref, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, ws, None) == -1
    assert L.moe_combine(ref, FAKE, FAKE, FAKE, None, None, None) == -1
    assert L.moe_combine(ref, FAKE_ODD, FAKE, FAKE, None, FAKE, None) == -1
    args = [ref, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, None, None, FAKE, None, FAKE, ws, None]
    assert L.moe_layer_forward(*args[:4], *args[4:11], None, *args[12:]) == -1     # out missing
    args_ws = list(args)
    args_ws[14] = ws - 256
    assert L.moe_layer_forward(*args_ws) == -3
    # shared expert requested but its weights missing
    s2 = abi.make_shape(W.CONFIGS["deepseek_v3"], num_tokens=16)
    ws2 = abi.moe_workspace_size(s2)
    assert L.moe_layer_forward(ctypes.byref(s2), FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, None, None,
                               FAKE, None, FAKE, ws2, None) == -1
    # replica map: no physical experts, missing tables or output
    assert L.moe_map_replicas(ref, FAKE, FAKE, FAKE, 0, FAKE, FAKE, ws, None) == -1
    assert L.moe_map_replicas(ref, FAKE, None, FAKE, 4, FAKE, FAKE, ws, None) == -1
    assert L.moe_map_replicas(ref, FAKE, FAKE, FAKE, 4, None, FAKE, ws, None) == -1
    assert L.moe_map_replicas(ref, FAKE, FAKE, FAKE, 4, FAKE, FAKE, ws - 1, None) == -3
    assert L.moe_group_score_sigmoid(FAKE, FAKE, -1, None) == -1
    assert L.moe_read_device_flags(None, None, None) == -1


def test_zero_tokens_is_a_no_op():
    L = abi.lib()
    s = base_shape(num_tokens=0)
    ws = abi.moe_workspace_size(s)
    ref = ctypes.byref(s)
    assert L.moe_route_topk(ref, FAKE, FAKE, None, None, None, None, FAKE, FAKE, FAKE, ws, None) == 0
    assert L.moe_dispatch(ref, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, ws, None) == 0
    assert L.moe_grouped_ffn(ref, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == 0
    assert L.moe_combine(ref, FAKE, FAKE, FAKE, None, FAKE, None) == 0
    assert L.moe_layer_forward(ref, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, None, None, FAKE, None,
                               FAKE, ws, None) == 0
    assert L.moe_map_replicas(ref, FAKE, FAKE, FAKE, 4, FAKE, FAKE, ws, None) == 0
    assert L.moe_group_score_sigmoid(FAKE, FAKE, 0, None) == 0


def test_binding_raises_on_error():
    with pytest.raises(abi.MoeError):
        abi.moe_workspace_size(base_shape(top_k=0))


def test_noalloc_entry_point_checks_before_any_hip_call():
    """The no-allocation layer call validates like moe_layer_forward, rejects
    shapes whose workspace exceeds its fixed device array, and enqueues
    nothing for zero tokens -- all before any HIP call."""
    L = abi.lib()
    assert abi.MOE_NOALLOC_SCRATCH_BYTES == 64 << 20
    header = open(HEADER).read()
    assert "#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)" in header

    def call(s, out=FAKE, wg=FAKE):
        return L.moe_layer_forward_noalloc(ctypes.byref(s), FAKE, FAKE, None, None, wg, FAKE, FAKE,
                                           FAKE, FAKE, FAKE, out, None, None)

    big = abi.make_shape(W.CONFIGS["mixtral_prefill"])            # 4096 tokens: ~400 MB of workspace
    assert abi.moe_workspace_size(big) > abi.MOE_NOALLOC_SCRATCH_BYTES
    assert call(big) == abi.MOE_ERR_WORKSPACE
    ds = abi.make_shape(W.CONFIGS["deepseek_v3"], num_tokens=1024)   # 289 MiB
    assert call(ds) == abi.MOE_ERR_WORKSPACE
    # decode-sized layers fit
    for name, T in (("mixtral_decode", 64), ("deepseek_v3", 64), ("qwen3_skewed", 512)):
        s = abi.make_shape(W.CONFIGS[name], num_tokens=T)
        assert abi.moe_workspace_size(s) <= abi.MOE_NOALLOC_SCRATCH_BYTES, name
    # argument errors come first, whatever the size
    assert call(big, out=None) == abi.MOE_ERR_INVALID_ARG
    assert call(abi.make_shape(W.CONFIGS["mixtral_decode"]), wg=FAKE_ODD) == abi.MOE_ERR_INVALID_ARG
    assert call(abi.make_shape(W.CONFIGS["mixtral_decode"], top_k=0)) == abi.MOE_ERR_INVALID_ARG
    # zero tokens: valid, nothing enqueued (no device is touched)
    assert call(abi.make_shape(W.CONFIGS["mixtral_decode"], num_tokens=0)) == abi.MOE_OK


def test_down_dtype_values():
    """down_dtype: 0 or act_dtype (weights in act_dtype) or MOE_F16 (bf16
    layers); MXFP8 layers take no fp16 down weights."""
    for dd in (0, abi.MOE_BF16, abi.MOE_F16):
        assert abi.moe_workspace_size(base_shape(down_dtype=dd)) > 0
    n = ctypes.c_size_t(0)
    s = base_shape(down_dtype=abi.MOE_F16)
    assert abi.lib().moe_workspace_size_mxfp8(ctypes.byref(s), ctypes.byref(n)) == abi.MOE_ERR_UNSUPPORTED
    L = abi.lib()
    assert L.moe_convert_bf16_to_f16(-1, FAKE, FAKE, None) == abi.MOE_ERR_INVALID_ARG
    assert L.moe_convert_bf16_to_f16(16, FAKE_ODD, FAKE, None) == abi.MOE_ERR_INVALID_ARG
    assert L.moe_convert_bf16_to_f16(0, None, None, None) == abi.MOE_OK


def test_mxfp8_scale_strides_bounded():
    """MXFP8 layers pass E*I (the gate/up weights' scale-word stride) as an
    int32; shapes beyond it are rejected, while the bf16 layer, whose offsets
    are 64-bit there, still takes them."""
    s = abi.make_shape(num_tokens=16, hidden=128, num_experts=512, intermediate=4194304, top_k=2)
    n = ctypes.c_size_t(0)
    assert abi.lib().moe_workspace_size_mxfp8(ctypes.byref(s), ctypes.byref(n)) == abi.MOE_ERR_UNSUPPORTED
    assert abi.lib().moe_workspace_size(ctypes.byref(s), ctypes.byref(n)) == abi.MOE_OK
    ok = abi.make_shape(num_tokens=16, hidden=128, num_experts=256, intermediate=4194304 - 128, top_k=2)
    assert abi.lib().moe_workspace_size_mxfp8(ctypes.byref(ok), ctypes.byref(n)) == abi.MOE_OK
