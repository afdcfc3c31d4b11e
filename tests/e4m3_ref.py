"""Library-side e4m3 tile quantisation for the CPU pins: torch's float8_e4m3fn
cast, with the tile scale formed through frexp / ldexp (the smallest power of
two at or above amax / 448, 1 for an all-zero tile), and the OCP MX E8M0
scale bytes (byte e stands for 2^(e - 127)) through numpy's frexp / ldexp."""
import numpy as np
import torch


def to_e8m0(s) -> np.ndarray:
    """Power-of-two scales (tensor or array) -> E8M0 bytes: s = 0.5 * 2^e by frexp."""
    s = s.numpy() if isinstance(s, torch.Tensor) else np.asarray(s)
    m, e = np.frexp(s.astype(np.float64))
    assert (m == 0.5).all(), "not a power of two"
    return (e - 1 + 127).astype(np.uint8)


def from_e8m0(b) -> np.ndarray:
    """E8M0 bytes -> fp64 scales 2^(b - 127)."""
    return np.ldexp(1.0, np.asarray(b).astype(np.int32) - 127)


def tile_scale(amax: torch.Tensor) -> torch.Tensor:
    """amax: float32 tensor -> float32 power-of-two scales."""
    t = amax.to(torch.float32) / 448.0
    m, e = torch.frexp(t)
    one = torch.ones_like(t)
    s = torch.where(m == 0.5, torch.ldexp(one, e - 1), torch.ldexp(one, e))
    return torch.where(amax > 0, s, one)


def quant_last(v: torch.Tensor):
    """1x128 tiles along the last dim: (codes as float8, scales float32 [..., n/128])."""
    v32 = v.to(torch.float32)
    t = v32.reshape(*v32.shape[:-1], -1, 128)
    s = tile_scale(t.abs().amax(-1))
    q = (t / s[..., None]).to(torch.float8_e4m3fn)
    return q.reshape(v32.shape), s
