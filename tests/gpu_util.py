"""Helpers for the GPU parity tests: host <-> device copies and error metrics."""
import sys
import time

import numpy as np
import torch

import synth


def dev(a: np.ndarray) -> torch.Tensor:
    """Host array -> cuda tensor with the same bytes (bf16 bits travel as int16)."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def empty(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="cuda")


def max_rel(a, r) -> float:
    """max |a - r| / max |r| (the error measure the tolerances are stated in)."""
    a = np.asarray(a, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = np.abs(r).max()
    return float(np.abs(a - r).max() / (den if den > 0 else 1.0))


def bf16v(a_u16: np.ndarray) -> np.ndarray:
    return synth.bf16_to_f32(a_u16)


# parity notes (near-tie and flip counts, errors) repeated in the session's
# terminal summary, where pytest shows them even for passing tests
NOTES = []


_T0 = time.time()


def say(*args):
    """Progress line that names the case (flushed before the GPU step runs),
    prefixed with the seconds since the session started."""
    msg = " ".join(str(a) for a in args)
    print(f"[{time.time() - _T0:7.1f}s] {msg}", flush=True)
    sys.stdout.flush()
    if any(w in msg for w in ("near-tie", "flipped", "max rel err", "bit-identical", "stage-wise")):
        NOTES.append(msg)


TOL = {"f32": 1e-4, "bf16": 2e-2, "e4m3": 5e-2}
NEAR_TIE = 1e-6


# The full-size prefill workloads (T=16384, d=7168, I=2048: about 23 GB of
# host inputs in bf16, 12 GB with e4m3 weights) take seconds to generate and
# several tests run each one; their inputs are generated once per session.
# The arrays are read-only, so no test can change what a later one sees.
_FULL = {}


def inputs_of(cfg):
    """synth.make_inputs(cfg), kept for the session when cfg is one of the
    full-size prefill workloads (synth.CONFIGS[4] or [5]) as defined."""
    if cfg not in (synth.CONFIGS[4], synth.CONFIGS[5]):
        return synth.make_inputs(cfg)
    key = cfg.name
    if key not in _FULL:
        inp = synth.make_inputs(cfg)
        for v in _walk(inp):
            v.flags.writeable = False
        _FULL[key] = inp
    return _FULL[key]


def _walk(obj):
    if isinstance(obj, np.ndarray):
        yield obj
    elif isinstance(obj, dict):
        for v in obj.values():
            yield from _walk(v)
