"""ctypes binding of libmoe.so (include/moe.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, passes their
device pointers and the current HIP stream to the C ABI, and raises MoeError
on a non-zero status.  No arithmetic of the layer happens here.  If the
library has not been built this module fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_EWORKSPACE, MOE_EHIP, MOE_ESCRATCH = range(6)
MOE_F32, MOE_BF16, MOE_E4M3 = 0, 1, 2
MOE_WS_DISPATCH, MOE_WS_FFN, MOE_WS_COMBINE, MOE_WS_ROUTE, MOE_WS_BACKWARD = 0, 1, 2, 3, 4
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "e4m3": MOE_E4M3}

EXPORTS = ("moe_route", "moe_dispatch", "moe_dispatch_noalloc", "moe_expert_ffn", "moe_expert_gate_up", "moe_expert_gate_up_rows",
           "moe_expert_down", "moe_combine", "moe_bias_update", "moe_backward", "moe_workspace_bytes",
           "moe_status_str")


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {msg}")
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("I", ctypes.c_int32), ("act", ctypes.c_int32), ("wt", ctypes.c_int32)]


class FfnWeights(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libmoe.so (raises if it is missing: build it first)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the HIP library first "
                           "(python -m sparse_expert_routing_amd.build); there is no CPU fallback")
    L = ctypes.CDLL(path)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    pd = ctypes.POINTER(Desc)
    pw = ctypes.POINTER(FfnWeights)
    L.moe_route.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_dispatch.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_dispatch_noalloc.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_expert_ffn.argtypes = [pd, vp, vp, vp, pw, vp, vp, sz, vp]
    L.moe_expert_gate_up.argtypes = [pd, vp, vp, vp, pw, vp, sz, vp]
    L.moe_expert_gate_up_rows.argtypes = [pd, vp, vp, vp, pw, vp, sz, vp]
    L.moe_expert_down.argtypes = [pd, vp, pw, vp, vp, sz, vp]
    L.moe_combine.argtypes = [pd, vp, pw, vp, vp, vp, vp, vp, sz, vp]
    L.moe_bias_update.argtypes = [pd, vp, f32, vp, vp]
    L.moe_backward.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, pw, pw, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                               vp, sz, vp]
    for fn in ("moe_route", "moe_dispatch", "moe_dispatch_noalloc", "moe_expert_ffn", "moe_expert_gate_up", "moe_expert_gate_up_rows",
               "moe_expert_down", "moe_combine", "moe_bias_update", "moe_backward"):
        getattr(L, fn).restype = ctypes.c_int
    L.moe_workspace_bytes.argtypes = [pd, i32]
    L.moe_workspace_bytes.restype = sz
    L.moe_status_str.argtypes = [ctypes.c_int]
    L.moe_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def desc(T, d, E, k, I, act="bf16", wt="bf16") -> Desc:
    return Desc(T, d, E, k, I, DTYPES[act], DTYPES[wt])


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, st):
    if st != MOE_OK:
        raise MoeError(fn, st, load().moe_status_str(st).decode())


def ffn_weights(gate, up, down, s_gate=None, s_up=None, s_down=None) -> FfnWeights:
    return FfnWeights(*[t.data_ptr() if t is not None else None for t in (gate, up, down, s_gate, s_up, s_down)])


def workspace_bytes(ds: Desc, stage: int) -> int:
    return load().moe_workspace_bytes(ctypes.byref(ds), stage)


def moe_route(ds, x, w_router, bias, idx, weights, gap=None, workspace=None, stream=None):
    nb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("moe_route", load().moe_route(ctypes.byref(ds), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(idx),
                                         _ptr(weights), _ptr(gap), _ptr(workspace), nb, _stream(stream)))


def moe_dispatch(ds, idx, x, counts, offsets, row_src, row_of, x_perm, x_perm_scale, workspace, stream=None):
    _check("moe_dispatch", load().moe_dispatch(
        ctypes.byref(ds), _ptr(idx), _ptr(x), _ptr(counts), _ptr(offsets), _ptr(row_src), _ptr(row_of),
        _ptr(x_perm), _ptr(x_perm_scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def moe_dispatch_noalloc(ds, idx, x, counts, offsets, row_src, row_of, x_perm, x_perm_scale, stream=None):
    _check("moe_dispatch_noalloc", load().moe_dispatch_noalloc(
        ctypes.byref(ds), _ptr(idx), _ptr(x), _ptr(counts), _ptr(offsets), _ptr(row_src), _ptr(row_of),
        _ptr(x_perm), _ptr(x_perm_scale), _stream(stream)))


def moe_expert_ffn(ds, x_perm, x_perm_scale, offsets, experts: FfnWeights, y_perm, workspace, stream=None):
    _check("moe_expert_ffn", load().moe_expert_ffn(
        ctypes.byref(ds), _ptr(x_perm), _ptr(x_perm_scale), _ptr(offsets), ctypes.byref(experts), _ptr(y_perm),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_expert_gate_up(ds, x_perm, x_perm_scale, offsets, experts: FfnWeights, workspace, stream=None):
    _check("moe_expert_gate_up", load().moe_expert_gate_up(
        ctypes.byref(ds), _ptr(x_perm), _ptr(x_perm_scale), _ptr(offsets), ctypes.byref(experts),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_expert_gate_up_rows(ds, x, row_src, offsets, experts: FfnWeights, workspace, stream=None):
    _check("moe_expert_gate_up_rows", load().moe_expert_gate_up_rows(
        ctypes.byref(ds), _ptr(x), _ptr(row_src), _ptr(offsets), ctypes.byref(experts),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_expert_down(ds, offsets, experts: FfnWeights, y_perm, workspace, stream=None):
    _check("moe_expert_down", load().moe_expert_down(
        ctypes.byref(ds), _ptr(offsets), ctypes.byref(experts), _ptr(y_perm), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_combine(ds, x, shared: FfnWeights, y_perm, row_of, weights, y, workspace, stream=None):
    _check("moe_combine", load().moe_combine(
        ctypes.byref(ds), _ptr(x), ctypes.byref(shared), _ptr(y_perm), _ptr(row_of), _ptr(weights), _ptr(y),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_backward(ds, x, w_router, idx, weights, offsets, row_src, row_of, experts: FfnWeights,
                 shared: FfnWeights, y_perm, dy, grads: dict, workspace, stream=None):
    """grads: device tensors dx, dw_router, dw_gate, dw_up, dw_down, ds_gate, ds_up, ds_down, and
    optionally dg (fp32, written)."""
    _check("moe_backward", load().moe_backward(
        ctypes.byref(ds), _ptr(x), _ptr(w_router), _ptr(idx), _ptr(weights), _ptr(offsets), _ptr(row_src),
        _ptr(row_of), ctypes.byref(experts), ctypes.byref(shared), _ptr(y_perm), _ptr(dy),
        *[_ptr(grads[n]) for n in ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "ds_gate", "ds_up",
                                    "ds_down")],
        _ptr(grads.get("dg")), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_bias_update(ds, counts, gamma, bias, stream=None):
    _check("moe_bias_update", load().moe_bias_update(ctypes.byref(ds), _ptr(counts), gamma, _ptr(bias),
                                                     _stream(stream)))
