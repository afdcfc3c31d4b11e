"""CPU oracle for the DeepSeekMoE layer with bias (auxiliary-loss-free) routing:
the forward, and the backward (gradients of the layer output).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
bench's ``cpu_baseline`` leg may import this package.  The product path (the
HIP library and its binding) never imports, links or calls it, and this
package imports nothing from the product path.

The arithmetic lives in ``moe_oracle.c`` (plain C loops, fp64 accumulation);
this module only marshals numpy arrays.  Every function cites the passage it
follows in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16, E4M3 = 0, 1, 2
_DT = {"f32": F32, "bf16": BF16, "e4m3": E4M3}


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("I", ctypes.c_int32), ("act", ctypes.c_int32),
                ("wt", ctypes.c_int32)]


class FFN(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("MOE_ORACLE_LIB")  # a mutant build, for the pin-strength test
        if not path:
            build(force=not os.path.exists(_LIB))
            path = _LIB
        L = ctypes.CDLL(path)
        vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        sig = {
            "oracle_route": [vp, vp, vp, vp, i64, vp, vp, vp, vp, vp],
            "oracle_choose": [i64, i32, i32, vp, vp, vp, vp, vp],
            "oracle_dispatch": [i32, i32, i32, vp, vp, vp, vp, vp],
            "oracle_bias_update": [i32, i32, i32, vp, f32, vp],
            "oracle_quant_e4m3_rows": [i64, i32, i32, vp, vp, vp],
            "oracle_expert_ffn": [vp, vp, vp, vp, vp, i64, vp, vp],
            "oracle_combine": [vp, vp, vp, vp, vp, vp, i64, vp, vp],
            "oracle_forward": [vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp],
            "oracle_backward": [vp] * 16 + [i32],
            "oracle_backward_shared_cols": [vp, vp, vp, vp, i32, vp, vp, vp, vp],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = None
        L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_decode.restype = ctypes.c_double
        L.oracle_bf16_encode.argtypes = [ctypes.c_float]
        L.oracle_bf16_encode.restype = ctypes.c_uint16
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_decode.restype = ctypes.c_double
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int32]
        L.oracle_set_threads.restype = None
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags.c_contiguous, "oracle inputs must be contiguous numpy arrays"
    return ctypes.c_void_p(a.ctypes.data)


def shape(T, d, E, k, I, act="bf16", wt="bf16") -> Shape:
    return Shape(T, d, E, k, I, _DT[act], _DT[wt])


def shape_of(cfg, T=None) -> Shape:
    return shape(cfg.T if T is None else T, cfg.d, cfg.E, cfg.k, cfg.I, cfg.act, cfg.wt)


def ffn(w: dict):
    """(FFN struct, keep-alive list) from a dict of gate/up/down (+ s_*) arrays."""
    keep = [w["gate"], w["up"], w["down"], w.get("s_gate"), w.get("s_up"), w.get("s_down")]
    return FFN(*[_p(a) for a in keep]), keep


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_threads(n: int) -> None:
    """Threads the oracle's later parallel regions use (from this thread)."""
    lib().oracle_set_threads(int(n))


def route(sh: Shape, x, wr, bias, tokens=None, want_s=False):
    """idx [n,k] int32 (ascending ids), g [n,k] f32, gap [n] f64, s [n,E] f64 or None."""
    n = sh.T if tokens is None else len(tokens)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    idx = np.empty((n, sh.k), np.int32)
    g = np.empty((n, sh.k), np.float32)
    gap = np.empty(n, np.float64)
    s = np.empty((n, sh.E), np.float64) if want_s else None
    lib().oracle_route(ctypes.byref(sh), _p(x), _p(wr), _p(bias), n, _p(tok), _p(idx), _p(g), _p(gap), _p(s))
    return idx, g, gap, s


def choose(s: np.ndarray, bias, k: int):
    """The choice alone from fp64 affinities s [n, E]: idx [n,k], g [n,k], gap [n]."""
    n, E = s.shape
    s = np.ascontiguousarray(s, dtype=np.float64)
    b = np.ascontiguousarray(bias, dtype=np.float32)
    idx = np.empty((n, k), np.int32)
    g = np.empty((n, k), np.float32)
    gap = np.empty(n, np.float64)
    lib().oracle_choose(n, E, k, _p(s), _p(b), _p(idx), _p(g), _p(gap))
    return idx, g, gap


def dispatch(idx: np.ndarray, E: int):
    """counts [E], offsets [E+1], row_src [T*k], row_of [T*k] (all int32)."""
    T, k = idx.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    row_src = np.empty(T * k, np.int32)
    row_of = np.empty(T * k, np.int32)
    lib().oracle_dispatch(T, E, k, _p(idx), _p(counts), _p(offsets), _p(row_src), _p(row_of))
    return counts, offsets, row_src, row_of


def bias_update(bias: np.ndarray, counts: np.ndarray, k: int, T: int, gamma: float = 1e-3) -> np.ndarray:
    """New fp32 bias (the input is not modified)."""
    b = np.array(bias, dtype=np.float32, copy=True)
    c = np.ascontiguousarray(counts, dtype=np.int32)
    lib().oracle_bias_update(len(b), k, T, _p(c), gamma, _p(b))
    return b


def quant_e4m3_rows(v: np.ndarray, in_dtype="bf16"):
    """1x128-tile e4m3 quantisation of rows: codes uint8 [rows, cols], scales as
    E8M0 bytes uint8 [rows, cols/128] (byte e stands for 2^(e - 127))."""
    rows, cols = v.shape
    v = np.ascontiguousarray(v)
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // 128), np.uint8)
    lib().oracle_quant_e4m3_rows(rows, cols, _DT[in_dtype], _p(v), _p(q), _p(s))
    return q, s


def expert_ffn(sh: Shape, experts: dict, offsets, a_rows, a_scales=None, rows=None):
    """Routed FFN on permuted rows: y_perm [n, d] (f32, or bf16 bits as uint16) for
    rows 0..T*k-1, or for the listed permuted rows (in list order)."""
    A = sh.T * sh.k
    n = A if rows is None else len(rows)
    rl = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    w, keep = ffn(experts)
    y = np.empty((n, sh.d), np.float32 if sh.wt == F32 else np.uint16)
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    lib().oracle_expert_ffn(ctypes.byref(sh), ctypes.byref(w), _p(offsets), _p(np.ascontiguousarray(a_rows)),
                            _p(a_scales), n, _p(rl), _p(y))
    del keep
    return y


def combine(sh: Shape, shared: dict, x, y_perm, row_of, g, tokens=None):
    """y [n, d] f32 = shared(x[t]) + sum_j g[t,j] * y_perm[row_of[t*k+j]]."""
    n = sh.T if tokens is None else len(tokens)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    w, keep = ffn(shared)
    y = np.empty((n, sh.d), np.float32)
    lib().oracle_combine(ctypes.byref(sh), ctypes.byref(w), _p(x), _p(y_perm),
                         _p(np.ascontiguousarray(row_of, dtype=np.int32)),
                         _p(np.ascontiguousarray(g, dtype=np.float32)), n, _p(tok), _p(y))
    del keep
    return y


def backward(sh: Shape, x, wr, idx, experts: dict, shared: dict, dy, weight_grads=True):
    """Gradients of the layer output for the routing idx [T,k] given dy [T,d] f32:
    dict of dx [T,d], dwr [E,d], dwg/dwu [E,I,d], dwd [E,d,I], dsg/dsu [I,d],
    dsd [d,I], dg [T,k] (all f32).  weight_grads=False: dx and dg only; an
    int e: dx, dg and routed expert e's dwr [1,d], dwg/dwu [1,I,d], dwd [1,d,I]
    (the sums over the given tokens only).  e4m3 weights: every backward GEMM
    on e4m3 operands (tiles along each GEMM's reduction; see the C source)."""
    T, d, E, k, I = sh.T, sh.d, sh.E, sh.k, sh.I
    we, k1 = ffn(experts)
    ws, k2 = ffn(shared)
    shp = dict(dx=(T, d), dwr=(E, d), dwg=(E, I, d), dwu=(E, I, d), dwd=(E, d, I), dsg=(I, d), dsu=(I, d),
               dsd=(d, I), dg=(T, k))
    one = not isinstance(weight_grads, bool)
    if one:
        assert 0 <= weight_grads < E
        shp.update(dwr=(1, d), dwg=(1, I, d), dwu=(1, I, d), dwd=(1, d, I), dsg=(1,), dsu=(1,), dsd=(1,))
    elif not weight_grads:
        shp = {n: (v if n in ("dx", "dg") else (1,)) for n, v in shp.items()}
    out = {n: np.empty(v, np.float32) for n, v in shp.items()}
    lib().oracle_backward(ctypes.byref(sh), _p(x), _p(np.ascontiguousarray(wr, dtype=np.float32)),
                          _p(np.ascontiguousarray(idx, dtype=np.int32)), ctypes.byref(we), ctypes.byref(ws),
                          _p(np.ascontiguousarray(dy, dtype=np.float32)),
                          *[_p(out[n]) for n in ("dx", "dwr", "dwg", "dwu", "dwd", "dsg", "dsu", "dsd", "dg")],
                          int(weight_grads) if one else (-1 if weight_grads else -2))
    del k1, k2
    if one:
        return {n: out[n] for n in ("dx", "dg", "dwr", "dwg", "dwu", "dwd")}
    return out if weight_grads else dict(dx=out["dx"], dg=out["dg"])


def backward_shared_cols(sh: Shape, x, shared: dict, dy, cols):
    """The shared expert's weight gradients for the SwiGLU columns `cols` only,
    over all sh.T tokens: dict of dsg, dsu [len(cols), d] (those rows of
    backward()'s dsg, dsu) and dsd [d, len(cols)] (those columns of its dsd),
    bit for bit what backward() gives there."""
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    nc = len(cols)
    ws, keep = ffn(shared)
    out = dict(dsg=np.empty((nc, sh.d), np.float32), dsu=np.empty((nc, sh.d), np.float32),
               dsd=np.empty((sh.d, nc), np.float32))
    lib().oracle_backward_shared_cols(ctypes.byref(sh), _p(x), ctypes.byref(ws),
                                      _p(np.ascontiguousarray(dy, dtype=np.float32)), nc, _p(cols),
                                      _p(out["dsg"]), _p(out["dsu"]), _p(out["dsd"]))
    del keep
    return out


def forward(sh: Shape, x, wr, bias, experts: dict, shared: dict, tokens=None):
    """Whole layer for a list of tokens: idx [n,k], g [n,k], gap [n], y [n,d] f32."""
    n = sh.T if tokens is None else len(tokens)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    we, k1 = ffn(experts)
    ws, k2 = ffn(shared)
    idx = np.empty((n, sh.k), np.int32)
    g = np.empty((n, sh.k), np.float32)
    gap = np.empty(n, np.float64)
    y = np.empty((n, sh.d), np.float32)
    lib().oracle_forward(ctypes.byref(sh), _p(x), _p(wr), _p(bias), ctypes.byref(we), ctypes.byref(ws), n,
                         _p(tok), _p(idx), _p(g), _p(gap), _p(y))
    del k1, k2
    return idx, g, gap, y


def bf16_encode(v: float) -> int:
    return lib().oracle_bf16_encode(v)


def bf16_decode(b: int) -> float:
    return lib().oracle_bf16_decode(b)


def e4m3_encode(v: float) -> int:
    return lib().oracle_e4m3_encode(v)


def e4m3_decode(c: int) -> float:
    return lib().oracle_e4m3_decode(c)


def e8m0_decode(e: int) -> float:
    return lib().oracle_e8m0_decode(e)
