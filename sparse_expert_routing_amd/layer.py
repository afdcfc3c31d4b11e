"""A DeepSeekMoE layer on one GPU: device buffers plus the five C-ABI calls.

torch is used for device memory and the stream only; each step of the layer
runs in the HIP kernels behind include/moe.h.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib

_TORCH_STORAGE = {"f32": torch.float32, "bf16": torch.int16, "e4m3": torch.uint8}


def _dev(a, device):
    """Host numpy array -> device tensor with the same bytes."""
    t = torch.from_numpy(a)
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.to(device, non_blocking=False)


class MoeLayer:
    """Weights and scratch of one layer; ``forward`` runs route -> dispatch ->
    expert FFN -> combine, ``update_bias`` the sign step, ``step`` both."""

    def __init__(self, T, d, I, act, wt, wr, experts: dict, shared: dict, E=256, k=8, device="cuda"):
        self.T, self.d, self.I, self.E, self.k = T, d, I, E, k
        self.act, self.wt = act, wt
        self.device = torch.device(device)
        self.desc = _lib.desc(T, d, E, k, I, act, wt)
        self.wr = _dev(wr, self.device)
        self.ex = {n: (_dev(a, self.device) if a is not None else None) for n, a in experts.items()}
        self.sh = {n: (_dev(a, self.device) if a is not None else None) for n, a in shared.items()}
        self.ex_w = _lib.ffn_weights(*(self.ex[n] for n in ("gate", "up", "down", "s_gate", "s_up", "s_down")))
        self.sh_w = _lib.ffn_weights(*(self.sh[n] for n in ("gate", "up", "down", "s_gate", "s_up", "s_down")))
        self._alloc()

    def _alloc(self):
        dev, T, d, E, k = self.device, self.T, self.d, self.E, self.k
        A = T * k
        i32 = dict(dtype=torch.int32, device=dev)
        self.idx = torch.empty((T, k), **i32)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.gap = torch.empty(T, dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.row_src = torch.empty(A, **i32)
        self.row_of = torch.empty(A, **i32)
        self.x_perm = self.x_perm_scale = None  # allocated on first use of the materialised dispatch
        self.y_perm = torch.empty((A, d), dtype=torch.float32 if self.wt == "f32" else torch.int16, device=dev)
        self.y = torch.empty((T, d), dtype=torch.float32, device=dev)
        ws = max(_lib.workspace_bytes(self.desc, s) for s in (0, 1, 2, 3))
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)

    def ensure_x_perm(self):
        if self.x_perm is None:
            A, d = self.T * self.k, self.d
            self.x_perm = torch.empty((A, d), dtype=_TORCH_STORAGE[self.wt], device=self.device)
            self.x_perm_scale = (torch.empty((A, d // 128), dtype=torch.uint8, device=self.device)
                                 if self.wt == "e4m3" else None)

    def forward(self, x, bias, gap=False, stream=None, gather_in_gemm=True):
        """One pass of the layer.  gather_in_gemm: the gate/up GEMM reads the
        token rows through row_src (no x_perm); otherwise moe_dispatch
        materialises x_perm and moe_expert_ffn consumes it.  Both give the
        same y bit for bit."""
        D = self.desc
        _lib.moe_route(D, x, self.wr, bias, self.idx, self.w, self.gap if gap else None, self.ws, stream)
        if gather_in_gemm:
            _lib.moe_dispatch(D, self.idx, x, self.counts, self.offsets, self.row_src, self.row_of, None, None,
                              self.ws, stream)
            _lib.moe_expert_gate_up_rows(D, x, self.row_src, self.offsets, self.ex_w, self.ws, stream)
            _lib.moe_expert_down(D, self.offsets, self.ex_w, self.y_perm, self.ws, stream)
        else:
            self.ensure_x_perm()
            _lib.moe_dispatch(D, self.idx, x, self.counts, self.offsets, self.row_src, self.row_of, self.x_perm,
                              self.x_perm_scale, self.ws, stream)
            _lib.moe_expert_ffn(D, self.x_perm, self.x_perm_scale, self.offsets, self.ex_w, self.y_perm, self.ws,
                                stream)
        _lib.moe_combine(D, x, self.sh_w, self.y_perm, self.row_of, self.w, self.y, self.ws, stream)
        return self.y

    def update_bias(self, bias, gamma=1e-3, stream=None):
        _lib.moe_bias_update(self.desc, self.counts, gamma, bias, stream)

    def step(self, x, bias, gamma=None, tokens_seen=0, stream=None):
        """One training step's forward and bias update; gamma defaults to the
        schedule's value for a step starting after `tokens_seen` tokens."""
        y = self.forward(x, bias, stream=stream)
        self.update_bias(bias, bias_gamma(tokens_seen) if gamma is None else gamma, stream)
        return y


# kbwen.com DeepSeek feed, "A bias term for each expert": the bias moves by
# 0.001 per step for the first 14.3T training tokens and by 0 for the rest.
# Reading: a step that starts before 14.3T tokens have been consumed uses
# 0.001.
GAMMA = 1e-3
GAMMA_TOKENS = 14.3e12


def bias_gamma(tokens_seen: float) -> float:
    """The bias step size for a training step that starts after `tokens_seen` tokens."""
    return GAMMA if tokens_seen < GAMMA_TOKENS else 0.0


def save_bias(path, bias) -> None:
    """Checkpoint the balancing state: the fp32 bias is the layer's only state
    that changes from step to step (DeepSeek V3 From Scratch, "In code":
    update_bias returns the new bias; kbwen.com DeepSeek feed, "A bias term
    for each expert").  Written as a .npy file holding the exact fp32 bits."""
    if isinstance(bias, torch.Tensor):
        bias = bias.detach().to("cpu").numpy()
    np.save(path, np.ascontiguousarray(bias, dtype=np.float32), allow_pickle=False)


def load_bias(path, device="cuda") -> torch.Tensor:
    """The bias saved by save_bias, as an fp32 tensor on `device` (bit-exact)."""
    b = np.load(path, allow_pickle=False)
    if b.dtype != np.float32 or b.ndim != 1:
        raise ValueError(f"{path}: expected a 1-D float32 bias, got {b.dtype} {b.shape}")
    return torch.from_numpy(b).to(device)


def layer_from_inputs(inp: dict, device="cuda") -> MoeLayer:
    """Build a layer from a synth.make_inputs() dict (weights uploaded once)."""
    c = inp["cfg"]
    return MoeLayer(c.T, c.d, c.I, c.act, c.wt, inp["wr"], inp["experts"], inp["shared"], c.E, c.k, device)


def upload(a, device="cuda"):
    return _dev(a, torch.device(device))
