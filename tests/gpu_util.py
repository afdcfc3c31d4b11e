"""Helpers for the GPU parity tests: host <-> device copies and error metrics."""
import sys

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


def say(*args):
    """Progress line that names the case (flushed before the GPU step runs)."""
    print(*args, flush=True)
    sys.stdout.flush()


TOL = {"f32": 1e-4, "bf16": 2e-2, "e4m3": 5e-2}
NEAR_TIE = 1e-6
