"""Checkpoint and resume of the balancing loop.

The per-expert bias is the only state the layer carries from one step to the
next (DeepSeek V3 From Scratch, "In code": update_bias maps the old bias and
the step's load to the new bias; kbwen.com DeepSeek feed, "A bias term for
each expert": the bias moves once per step).  So 50 steps, a save and reload
of the fp32 bias, and 50 more steps must equal 100 straight steps, bit for
bit: on the CPU with the oracle's loop (and the package's save/load helpers),
and on the GPU through the C ABI with a layer object built afresh after the
reload."""
import numpy as np
import pytest

import oracle
import synth
from sparse_expert_routing_amd.layer import load_bias, save_bias

CFG = synth.CONFIGS[4].with_(T=2048, d=1024, I=256)  # the skewed workload's recipe, reduced


def oracle_loop(s, bias, steps, k, T, gamma):
    b = np.array(bias, dtype=np.float32)
    counts = []
    for _ in range(steps):
        idx, _, _ = oracle.choose(s, b, k)
        c = oracle.dispatch(idx, s.shape[1])[0]
        counts.append(c)
        b = oracle.bias_update(b, c, k, T, gamma)
    return b, counts


def test_resume_oracle_loop(tmp_path):
    cfg = CFG
    inp = synth.make_inputs(cfg)
    _, _, _, s = oracle.route(oracle.shape_of(cfg), inp["x"], inp["wr"], inp["bias"], want_s=True)
    b100, c100 = oracle_loop(s, inp["bias"], 100, cfg.k, cfg.T, cfg.gamma)
    b50, c50 = oracle_loop(s, inp["bias"], 50, cfg.k, cfg.T, cfg.gamma)
    path = tmp_path / "bias.npy"
    save_bias(path, b50)
    b_re = load_bias(path, device="cpu").numpy()
    assert np.array_equal(b_re.view(np.uint32), b50.view(np.uint32))
    b_end, c_rest = oracle_loop(s, b_re, 50, cfg.k, cfg.T, cfg.gamma)
    assert np.array_equal(b_end.view(np.uint32), b100.view(np.uint32))
    assert all(np.array_equal(a, b) for a, b in zip(c100, c50 + c_rest))
    assert not np.array_equal(b100, inp["bias"])  # the loop did move the bias


@pytest.mark.gpu
def test_resume_gpu_layer(tmp_path):
    import torch

    from sparse_expert_routing_amd import _lib
    from sparse_expert_routing_amd.layer import layer_from_inputs, upload
    from tests.gpu_util import host, say
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    cfg = CFG
    inp = synth.make_inputs(cfg)
    say(f"[resume] {cfg.name}: 100 straight whole-layer steps")
    layer = layer_from_inputs(inp)
    x = upload(inp["x"])
    b = upload(inp["bias"])
    c100 = []
    for _ in range(100):
        layer.step(x, b, gamma=cfg.gamma)
        c100.append(layer.counts.clone())
    b100 = host(b).copy()
    say(f"[resume] {cfg.name}: 50 steps, save, fresh layer, reload, 50 steps")
    b = upload(inp["bias"])
    c_resumed = []
    for _ in range(50):
        layer.step(x, b, gamma=cfg.gamma)
        c_resumed.append(layer.counts.clone())
    path = tmp_path / "bias.npy"
    save_bias(path, b)
    del layer, b
    layer = layer_from_inputs(inp)
    b = load_bias(path)
    for _ in range(50):
        layer.step(x, b, gamma=cfg.gamma)
        c_resumed.append(layer.counts.clone())
    torch.cuda.synchronize()
    assert np.array_equal(host(b).view(np.uint32), b100.view(np.uint32))
    assert all(torch.equal(a, r) for a, r in zip(c100, c_resumed))
