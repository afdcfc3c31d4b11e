"""The layer step under HIP graph capture.  No call of the library allocates,
synchronises or records a memset, so one loop step (forward + bias update)
can be captured once and replayed: each replay must equal the same step of
the eager loop bit for bit (the bias evolves in place from replay to replay).
Between the replays the program does eager work of its own and synchronises,
and every replay is checked, not only the first."""
import pytest
import torch

import synth
from sparse_expert_routing_amd import _lib
from sparse_expert_routing_amd.layer import layer_from_inputs, upload
from tests.gpu_util import inputs_of, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


CASES = {
    "mid": lambda: synth.CONFIGS[2],
    "skewed-reduced": lambda: synth.CONFIGS[4].with_(name="prefill-zipf-bf16 T4096 d1024 I512", T=4096, d=1024,
                                                     I=512),
    "fp8-full": lambda: synth.CONFIGS[5],
}


@pytest.mark.parametrize("case", list(CASES))
def test_layer_step_replays_from_a_hip_graph(case):
    cfg = CASES[case]()
    steps = 4
    say(f"[graph] {cfg.name}: {steps} eager loop steps, then one captured step replayed {steps} times")
    inp = inputs_of(cfg)
    layer = layer_from_inputs(inp)
    x = upload(inp["x"])

    b = upload(inp["bias"])
    eager = []
    for _ in range(steps):
        layer.forward(x, b)
        layer.update_bias(b, cfg.gamma)
        torch.cuda.synchronize()
        eager.append(dict(y=layer.y.clone(), bias=b.clone(), counts=layer.counts.clone(), idx=layer.idx.clone()))

    b = upload(inp["bias"])
    scratch_bias = b.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up before capture, on a bias of its own
        layer.forward(x, scratch_bias)
        layer.update_bias(scratch_bias, cfg.gamma)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, b)
        layer.update_bias(b, cfg.gamma)
    torch.cuda.synchronize()
    for s in range(steps):
        g.replay()
        torch.cuda.synchronize()
        other = torch.arange(1 << 20, device="cuda", dtype=torch.float32).mul_(0.5).sum()  # eager work
        torch.cuda.synchronize()
        assert float(other) > 0
        for n, ref in eager[s].items():
            got = {"y": layer.y, "bias": b, "counts": layer.counts, "idx": layer.idx}[n]
            assert torch.equal(_bits(got), _bits(ref)), f"{cfg.name}: replay {s}: {n} differs from the eager step"
    say(f"[graph] {cfg.name}: every replay bit-identical to its eager step")
