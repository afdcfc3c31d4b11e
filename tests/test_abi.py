"""The C ABI library on the CPU: it loads, exports every function include/moe.h
declares, and rejects invalid arguments on the host with the documented
status codes before anything reaches a GPU (all calls here fail validation,
so no kernel is launched)."""
import ctypes
import os
import re

import pytest

import sparse_expert_routing_amd as moe
from sparse_expert_routing_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", hdr)))


def test_header_declares_the_five_calls():
    fns = declared_functions()
    for f in ("moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_bias_update"):
        assert f in fns
    assert set(fns) == set(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib.load()
    for f in declared_functions():
        assert hasattr(L, f), f


def good_desc(**kw):
    d = dict(T=64, d=256, E=256, k=8, I=128, act="bf16", wt="bf16")
    d.update(kw)
    return _lib.desc(**d)


def call_route(ds, ptrs=True):
    p = ctypes.c_void_p(0x1000) if ptrs else None
    return _lib.load().moe_route(ctypes.byref(ds), p, p, p, p, p, None, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), _lib.MOE_EINVAL), (dict(d=-64), _lib.MOE_EINVAL), (dict(k=300), _lib.MOE_EINVAL),
    (dict(E=128), _lib.MOE_ENOTSUP), (dict(k=6), _lib.MOE_ENOTSUP), (dict(d=96), _lib.MOE_ENOTSUP),
    (dict(I=100), _lib.MOE_ENOTSUP), (dict(act="f32", wt="bf16"), _lib.MOE_ENOTSUP),
    (dict(wt="e4m3", d=192), _lib.MOE_EINVAL), (dict(wt="e4m3", I=64), _lib.MOE_EINVAL),
    (dict(act="e4m3", wt="e4m3"), _lib.MOE_ENOTSUP), (dict(d=192), _lib.MOE_ENOTSUP),
    (dict(T=1 << 28), _lib.MOE_ENOTSUP),  # T*k = 2^31: the routed rows' int32 indices
])
def test_shape_validation(kw, status):
    assert call_route(good_desc(**kw)) == status
    assert _lib.workspace_bytes(good_desc(**kw), 0) == 0


def test_null_pointers_rejected():
    assert call_route(good_desc(), ptrs=False) == _lib.MOE_EINVAL
    L = _lib.load()
    ds = good_desc()
    assert L.moe_route(None, None, None, None, None, None, None, None, 0, None) == _lib.MOE_EINVAL
    assert L.moe_bias_update(ctypes.byref(ds), None, ctypes.c_float(1e-3), None, None) == _lib.MOE_EINVAL
    w = _lib.FfnWeights(0x1000, 0x1000, None, None, None, None)  # missing down
    p = ctypes.c_void_p(0x1000)
    assert L.moe_expert_ffn(ctypes.byref(ds), p, None, p, ctypes.byref(w), p, p, 1 << 30, None) == _lib.MOE_EINVAL
    ds8 = good_desc(wt="e4m3")
    w8 = _lib.FfnWeights(0x1000, 0x1000, 0x1000, None, None, None)  # e4m3 without scales
    assert L.moe_expert_ffn(ctypes.byref(ds8), p, p, p, ctypes.byref(w8), p, p, 1 << 30, None) == _lib.MOE_EINVAL


def test_small_workspace_rejected():
    L = _lib.load()
    ds = good_desc()
    p = ctypes.c_void_p(0x1000)
    need_r = _lib.workspace_bytes(ds, _lib.MOE_WS_ROUTE)
    assert need_r >= 3 * 256 * 256 * 2 + 64 * 256 * 4  # bf16 router split + fp32 logits
    assert call_route(ds) == _lib.MOE_EWORKSPACE
    assert L.moe_route(ctypes.byref(ds), p, p, p, p, p, None, p, need_r - 1, None) == _lib.MOE_EWORKSPACE
    assert _lib.workspace_bytes(good_desc(act="f32", wt="f32"), _lib.MOE_WS_ROUTE) == 0
    need = _lib.workspace_bytes(ds, _lib.MOE_WS_DISPATCH)
    assert need > 0
    st = L.moe_dispatch(ctypes.byref(ds), p, p, p, p, p, p, p, None, p, need - 1, None)
    assert st == _lib.MOE_EWORKSPACE
    w = _lib.FfnWeights(0x1000, 0x1000, 0x1000, None, None, None)
    need = _lib.workspace_bytes(ds, _lib.MOE_WS_FFN)
    assert L.moe_expert_ffn(ctypes.byref(ds), p, None, p, ctypes.byref(w), p, p, need - 1, None) == _lib.MOE_EWORKSPACE
    need = _lib.workspace_bytes(ds, _lib.MOE_WS_COMBINE)
    assert L.moe_combine(ctypes.byref(ds), p, ctypes.byref(w), p, p, p, p, p, need - 1, None) == _lib.MOE_EWORKSPACE


def test_workspace_sizes_grow_with_shape():
    small = good_desc(T=64)
    big = good_desc(T=16384, d=7168, I=2048)
    for s in range(3):
        assert _lib.workspace_bytes(big, s) > _lib.workspace_bytes(small, s) > 0
    # FFN scratch holds h: T*k rows of I values in the GEMM input type
    assert _lib.workspace_bytes(big, 1) >= 16384 * 8 * 2048 * 2


def test_status_strings():
    L = _lib.load()
    for s in range(5):
        assert L.moe_status_str(s).decode().startswith("MOE_")


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "sparse_expert_routing_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f"{f} mentions the oracle"


def test_dispatch_noalloc_limit_checked_before_launch():
    """More tokens than the static scratch holds: MOE_ESCRATCH from the host
    check, before any device work."""
    L = _lib.load()
    p = ctypes.c_void_p(0x1000)
    ds = good_desc(T=(1 << 20) + 1)
    assert L.moe_dispatch_noalloc(ctypes.byref(ds), p, p, p, p, p, p, None, None, None) == _lib.MOE_ESCRATCH
    assert L.moe_dispatch_noalloc(ctypes.byref(good_desc()), None, p, p, p, p, p, None, None, None) == _lib.MOE_EINVAL
    assert L.moe_status_str(_lib.MOE_ESCRATCH).decode().startswith("MOE_ESCRATCH")
