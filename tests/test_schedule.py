"""The balancing loop's control variants on the host: the bias step-size
schedule (kbwen.com DeepSeek feed, "A bias term for each expert": 0.001 for
the first 14.3T training tokens, 0 afterwards), the identity step at
gamma 0, and the fresh per-step batches of the synthetic workload."""
import numpy as np

import oracle
import synth
from sparse_expert_routing_amd.layer import GAMMA, GAMMA_TOKENS, bias_gamma


def test_gamma_schedule():
    assert GAMMA == 1e-3 and GAMMA_TOKENS == 14.3e12
    assert bias_gamma(0) == 1e-3
    assert bias_gamma(14.3e12 - 16384) == 1e-3
    assert bias_gamma(14.3e12) == 0.0
    assert bias_gamma(14.8e12) == 0.0


def test_gamma_zero_step_is_identity():
    rng = np.random.default_rng(5)
    T, k, E = 1000, 8, 256
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    counts = np.bincount(rng.integers(0, E, T * k), minlength=E).astype(np.int32)
    nb = oracle.bias_update(b, counts, k, T, 0.0)
    assert np.array_equal(nb.view(np.uint32), b.view(np.uint32))
    moved = oracle.bias_update(b, counts, k, T, 1e-3)
    assert not np.array_equal(moved, b)  # the same loads do move it at 0.001


def test_fresh_batches_are_distinct_and_deterministic():
    cfg = synth.CONFIGS[4].with_(T=64, d=256, I=64)
    x0 = synth.make_x_step(cfg, 0)
    assert np.array_equal(x0, synth.make_router(cfg)[0])
    x1, x1b, x2 = synth.make_x_step(cfg, 1), synth.make_x_step(cfg, 1), synth.make_x_step(cfg, 2)
    assert np.array_equal(x1, x1b)
    assert not np.array_equal(x1, x0) and not np.array_equal(x1, x2)
    assert x1.dtype == x0.dtype and x1.shape == x0.shape
