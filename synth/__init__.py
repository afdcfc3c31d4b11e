"""Seeded synthetic inputs for the MoE layer (shared by the oracle side and the HIP side).

This module draws numbers and stores them in a tensor's storage format; it
holds none of the layer's arithmetic.  Values depend only on
(seed, tensor id, element index), never on thread count, so the same call
gives the same bytes on any host.

The five workloads (``CONFIGS``) follow the DeepSeek-V3 MoE shape the pages
describe -- 256 routed experts plus one shared expert, top-8 routing (DeepSeek
V3 From Scratch, "The idea"; crackai.dev DeepSeek-V3 summary, "How It Works")
-- with d_model, expert width, dtypes, distributions and seeds of our own
choosing for each workload (tiny fp32, mid bf16, decode bf16, skewed prefill
bf16 with a 100-step balancing loop, prefill fp8).  A sixth workload stands
for one GPU's share of an 8-way expert-parallel layer: the bias confines the
choice to 32 experts, so the grouped GEMMs see 32 groups of about 4096 rows
each, the shape one of 8 GPUs holding 32 experts each would run.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# tensor ids (part of the Philox key)
TID_X, TID_WR, TID_BIAS = 1, 2, 3
TID_GATE, TID_UP, TID_DOWN = 4, 5, 6
TID_SGATE, TID_SUP, TID_SDOWN = 7, 8, 9
TID_IDS = 10
TID_AUX = 11
TID_XSTEP = 100  # fresh batches of the balancing loop: step s >= 1 draws x from id 100 + s

F32, BF16, E4M3 = "f32", "bf16", "e4m3"


def build(force: bool = True) -> str:
    """Compile gen.c into libsynth.so next to it (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-msse4.2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=not os.path.exists(_LIB))
        L = ctypes.CDLL(_LIB)
        u64, u32, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_double, ctypes.c_void_p)
        L.synth_philox4x64_10.argtypes = [vp, vp, vp]
        L.synth_normal.argtypes = [u64, u32, i64, dbl, i32, vp]
        L.synth_normal_rowpow.argtypes = [u64, u32, i64, i64, dbl, dbl, vp]
        L.synth_uniform.argtypes = [u64, u32, i64, dbl, dbl, vp]
        L.synth_normal_e4m3_blocks.argtypes = [u64, u32, i64, i64, i64, dbl, vp, vp]
        L.synth_random_ids.argtypes = [u64, u32, i64, i32, i32, vp]
        L.synth_e4m3_encode.argtypes = [i64, vp, vp]
        for f in ("synth_philox4x64_10", "synth_normal", "synth_normal_rowpow", "synth_uniform",
                  "synth_normal_e4m3_blocks", "synth_random_ids", "synth_e4m3_encode"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return ctypes.c_void_p(a.ctypes.data)


def philox4x64_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint64)
    k = np.asarray(key, dtype=np.uint64)
    out = np.zeros(4, dtype=np.uint64)
    lib().synth_philox4x64_10(_p(c), _p(k), _p(out))
    return out


def normal(seed, tensor, shape, std, dtype=F32):
    n = int(np.prod(shape))
    if dtype == F32:
        out = np.empty(shape, dtype=np.float32)
        lib().synth_normal(seed, tensor, n, std, 0, _p(out))
    elif dtype == BF16:
        out = np.empty(shape, dtype=np.uint16)
        lib().synth_normal(seed, tensor, n, std, 1, _p(out))
    else:
        raise ValueError(dtype)
    return out


def normal_rowpow(seed, tensor, rows, cols, std, s):
    out = np.empty((rows, cols), dtype=np.float32)
    lib().synth_normal_rowpow(seed, tensor, rows, cols, std, s, _p(out))
    return out


def uniform(seed, tensor, n, lo, hi):
    out = np.empty(n, dtype=np.float32)
    lib().synth_uniform(seed, tensor, n, lo, hi, _p(out))
    return out


def normal_e4m3_blocks(seed, tensor, G, R, C, std):
    assert R % 128 == 0 and C % 128 == 0
    q = np.empty((G, R, C), dtype=np.uint8)
    s = np.empty((G, R // 128, C // 128), dtype=np.uint8)  # E8M0 bytes: 2^(s - 127)
    lib().synth_normal_e4m3_blocks(seed, tensor, G, R, C, std, _p(q), _p(s))
    return q, s


def random_ids(seed, tensor, T, E, k):
    out = np.empty((T, k), dtype=np.int32)
    lib().synth_random_ids(seed, tensor, T, E, k, _p(out))
    return out


def e4m3_encode(values: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().synth_e4m3_encode(v.size, _p(v), _p(out))
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seed: int
    T: int
    d: int
    I: int
    act: str = BF16          # dtype of x
    wt: str = BF16           # dtype of expert weights (and of the expert GEMM inputs)
    bias: str = "uniform"    # "zero", "uniform" (U(-0.05, 0.05)) or "shard32" (1 for experts 0-31, else 0)
    skew: float = 0.0        # router row power-law exponent (0 = none)
    steps: int = 1           # forward + bias-update steps of the balancing loop
    E: int = 256
    k: int = 8
    std_x: float = 1.0
    std_w: float = 0.02
    gamma: float = 1e-3

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    @property
    def A(self) -> int:
        return self.T * self.k


CONFIGS = {
    1: Config("tiny-f32 T32 d256 I64", seed=0, T=32, d=256, I=64, act=F32, wt=F32, bias="zero"),
    2: Config("mid-bf16 T2048 d2048 I512", seed=1, T=2048, d=2048, I=512),
    3: Config("decode-bf16 T64 d7168 I2048", seed=2, T=64, d=7168, I=2048),
    4: Config("prefill-zipf-bf16 T16384 d7168 I2048", seed=3, T=16384, d=7168, I=2048,
              bias="zero", skew=1.1, steps=100),
    5: Config("prefill-fp8 T16384 d7168 I2048", seed=4, T=16384, d=7168, I=2048, wt=E4M3),
    # one GPU's share of an 8-way expert-parallel layer (32 local experts)
    6: Config("ep8-shard-bf16 T16384 d7168 I2048 E32", seed=5, T=16384, d=7168, I=2048, bias="shard32"),
}


def make_router(cfg: Config):
    """x, router matrix and initial bias (host numpy arrays)."""
    x = normal(cfg.seed, TID_X, (cfg.T, cfg.d), cfg.std_x, BF16 if cfg.act == BF16 else F32)
    if cfg.skew:
        wr = normal_rowpow(cfg.seed, TID_WR, cfg.E, cfg.d, cfg.std_w, cfg.skew)
    else:
        wr = normal(cfg.seed, TID_WR, (cfg.E, cfg.d), cfg.std_w, F32)
    if cfg.bias == "zero":
        bias = np.zeros(cfg.E, dtype=np.float32)
    elif cfg.bias == "shard32":
        # a sigmoid affinity lies in (0, 1): a bias of 1 on experts 0-31 puts
        # every token's top 8 among them
        bias = np.where(np.arange(cfg.E) < 32, 1.0, 0.0).astype(np.float32)
    else:
        bias = uniform(cfg.seed, TID_BIAS, cfg.E, -0.05, 0.05)
    return x, wr, bias


def make_ffn(cfg: Config, G: int, tids):
    """Weights of G SwiGLU experts: gate, up [G, I, d] and down [G, d, I], plus
    128x128 block scales (E8M0 bytes) when stored as e4m3 (None otherwise)."""
    tg, tu, td = tids
    if cfg.wt == E4M3:
        g, sg = normal_e4m3_blocks(cfg.seed, tg, G, cfg.I, cfg.d, cfg.std_w)
        u, su = normal_e4m3_blocks(cfg.seed, tu, G, cfg.I, cfg.d, cfg.std_w)
        dn, sd = normal_e4m3_blocks(cfg.seed, td, G, cfg.d, cfg.I, cfg.std_w)
        return dict(gate=g, up=u, down=dn, s_gate=sg, s_up=su, s_down=sd)
    dt = BF16 if cfg.wt == BF16 else F32
    return dict(gate=normal(cfg.seed, tg, (G, cfg.I, cfg.d), cfg.std_w, dt),
                up=normal(cfg.seed, tu, (G, cfg.I, cfg.d), cfg.std_w, dt),
                down=normal(cfg.seed, td, (G, cfg.d, cfg.I), cfg.std_w, dt),
                s_gate=None, s_up=None, s_down=None)


def make_x_step(cfg: Config, step: int):
    """The token batch of balancing-loop step `step` when every step takes a
    fresh batch: step 0 is the workload's x, step s >= 1 the same
    distribution under tensor id TID_XSTEP + s (host array)."""
    if step == 0:
        return make_router(cfg)[0]
    return normal(cfg.seed, TID_XSTEP + step, (cfg.T, cfg.d), cfg.std_x, BF16 if cfg.act == BF16 else F32)


def make_inputs(cfg: Config) -> dict:
    """All inputs of one workload as host arrays (bf16 as uint16 bits, e4m3 as uint8 codes)."""
    x, wr, bias = make_router(cfg)
    return dict(cfg=cfg, x=x, wr=wr, bias=bias,
                experts=make_ffn(cfg, cfg.E, (TID_GATE, TID_UP, TID_DOWN)),
                shared=make_ffn(cfg, 1, (TID_SGATE, TID_SUP, TID_SDOWN)))
