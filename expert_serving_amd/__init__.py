"""MI355X (gfx950) MoE-layer forward: router, dispatch, grouped SwiGLU FFN, combine.

The compute path is the HIP library `libmoe_mi355x.so` behind the C ABI in
`include/moe_mi355x.h`; `abi` binds it with ctypes.  PyTorch only supplies
device memory and streams.
"""

from . import abi  # noqa: F401
from .abi import (moe_combine, moe_dispatch, moe_grouped_ffn, moe_layer_forward,  # noqa: F401
                  moe_read_device_flags, moe_route_topk, moe_workspace_size, make_shape)
