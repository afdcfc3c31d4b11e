"""The seeded input generator: known answers, determinism, thread independence."""
import hashlib
import os
import subprocess
import sys

import numpy as np
import torch

import synth
from tests import e4m3_ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _inc(ctr):
    """numpy's Philox increments its 256-bit counter before each block."""
    c = [int(v) for v in ctr]
    for i in range(4):
        c[i] = (c[i] + 1) % 2**64
        if c[i] != 0:
            break
    return c


def test_philox_matches_numpy_bit_generator():
    cases = [((0, 0), (0, 0, 0, 0)), ((123456789, 987654321), (5, 7, 11, 13)),
             ((2**64 - 1, 2**63 + 5), (2**64 - 1, 2**64 - 1, 3, 4))]
    for key, ctr in cases:
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
        ref = bg.random_raw(4).astype(np.uint64)
        assert np.array_equal(synth.philox4x64_10(_inc(ctr), key), ref)


def test_normals_have_the_stated_moments():
    v = synth.bf16_to_f32(synth.normal(9, 4, (1 << 20,), 0.02, "bf16")).astype(np.float64)
    assert abs(v.mean()) < 1e-4 and abs(v.std() - 0.02) < 1e-4
    f = synth.normal(9, 5, (1 << 18,), 1.0, "f32").astype(np.float64)
    assert abs(f.mean()) < 1e-2 and abs(f.std() - 1.0) < 1e-2
    u = synth.uniform(9, 6, 1 << 18, -0.05, 0.05)
    assert u.min() >= -0.05 and u.max() < 0.05 and abs(u.mean()) < 1e-3


def test_e4m3_weights_are_the_bf16_draws_quantised():
    q, s = synth.normal_e4m3_blocks(7, 4, 2, 256, 384, 0.02)
    b = synth.normal(7, 4, (2, 256, 384), 0.02, "bf16")
    v = torch.from_numpy(synth.bf16_to_f32(b)).reshape(2, 2, 128, 3, 128)
    amax = v.abs().amax(dim=(2, 4))
    sc = e4m3_ref.tile_scale(amax)
    assert s.dtype == np.uint8 and np.array_equal(s, e4m3_ref.to_e8m0(sc))
    ref = (v / sc[:, :, None, :, None]).to(torch.float8_e4m3fn)
    assert np.array_equal(q, ref.view(torch.uint8).reshape(2, 256, 384).numpy())


def test_generator_encoder_matches_torch():
    rng = np.random.default_rng(3)
    v = (rng.uniform(-448, 448, 50000) * rng.choice([1, 1e-2, 1e-4], 50000)).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(synth.e4m3_encode(v), ref)


def test_random_ids_distinct_sorted():
    idx = synth.random_ids(1, synth.TID_IDS, 1000, 256, 8)
    assert np.all(np.diff(idx, axis=1) > 0) and idx.min() >= 0 and idx.max() < 256
    counts = np.bincount(idx.ravel(), minlength=256)
    assert counts.min() > 0


def _digest():
    x = synth.normal(3, 1, (4096, 96), 1.0, "bf16")
    w = synth.normal(3, 2, (1000, 33), 0.02, "f32")
    q, s = synth.normal_e4m3_blocks(3, 4, 1, 128, 256, 0.02)
    h = hashlib.sha256()
    for a in (x, w, q, s):
        h.update(a.tobytes())
    return h.hexdigest()


def test_values_do_not_depend_on_thread_count():
    code = "import synth, tests.test_synth as t; print(t._digest())"
    outs = []
    for n in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=n, PYTHONPATH=ROOT)
        outs.append(subprocess.check_output([sys.executable, "-c", code], cwd=ROOT, env=env, text=True).strip())
    assert outs[0] == outs[1] == _digest()


def test_shard_workload_confines_the_choice_to_32_experts():
    """The expert-parallel shard workload: its bias puts every token's top 8
    among experts 0-31, with every one of them used (checked on the oracle's
    routing of a reduced copy)."""
    import oracle
    cfg = synth.CONFIGS[6].with_(T=512, d=512)
    x, wr, bias = synth.make_router(cfg)
    assert np.array_equal(bias[:32], np.ones(32, np.float32)) and not bias[32:].any()
    idx, _, _, _ = oracle.route(oracle.shape_of(cfg), x, wr, bias)
    counts = np.bincount(idx.ravel(), minlength=256)
    assert counts[32:].sum() == 0 and (counts[:32] > 0).all()
