"""MI355X (gfx950) DeepSeekMoE layer forward with auxiliary-loss-free routing.

The layer runs in hand-written HIP kernels behind a C ABI (include/moe.h);
this package holds those sources (csrc/), the in-tree build (build.py), the
ctypes binding (_lib.py) and a thin layer object (layer.py).
"""
from . import _lib  # noqa: F401
from ._lib import (MoeError, desc, ffn_weights, moe_backward, moe_bias_update, moe_combine,  # noqa: F401
                   moe_dispatch, moe_expert_down, moe_expert_ffn, moe_expert_gate_up, moe_expert_gate_up_rows,
                   moe_route, workspace_bytes)
