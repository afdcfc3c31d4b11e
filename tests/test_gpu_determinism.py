"""Run-to-run determinism of the layer at the full-size prefill workloads,
in the launch configuration bench.py times.  Ids, counts and permutations
must be bit-exact (the dispatch decides order by token masks and popcounts,
never by atomics; the GEMMs, the combine and the split-K sums add in a fixed
order), so two runs in one process must agree bit for bit in every output,
including the floating-point ones.  Between the runs every output and the
workspace are overwritten with 0xFF bytes, so no result can come from the
previous run's memory."""
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


@pytest.mark.parametrize("cid", [4, 5])
def test_layer_bitwise_deterministic_full_size(cid):
    cfg = synth.CONFIGS[cid]
    say(f"[determinism] {cfg.name}: two forward + bias steps")
    inp = inputs_of(cfg)
    layer = layer_from_inputs(inp)
    x = upload(inp["x"])
    runs = []
    for r in range(2):
        b = upload(inp["bias"])
        for t in (layer.idx, layer.w, layer.gap, layer.counts, layer.offsets, layer.row_src, layer.row_of,
                  layer.y_perm, layer.y, layer.ws):
            t.view(torch.uint8).fill_(0xFF)
        layer.forward(x, b, gap=True)
        layer.update_bias(b, cfg.gamma)
        torch.cuda.synchronize()
        runs.append(dict(idx=layer.idx.clone(), w=layer.w.clone(), gap=layer.gap.clone(),
                         counts=layer.counts.clone(), offsets=layer.offsets.clone(),
                         row_src=layer.row_src.clone(), row_of=layer.row_of.clone(),
                         y_perm=layer.y_perm.clone(), y=layer.y.clone(), bias=b.clone()))
    for n in runs[0]:
        assert torch.equal(_bits(runs[0][n]), _bits(runs[1][n])), f"{cfg.name}: {n} differs between runs"
    say(f"[determinism] {cfg.name}: every output bit-identical")


@pytest.mark.parametrize("cid", [2, 4])
def test_layer_on_a_side_stream(cid):
    """Every kernel is launched on the caller's stream: the layer run on a
    non-default stream, with only that stream synchronised, equals the
    default-stream run bit for bit (the mid workload on the small-tile
    kernels; the skewed prefill workload at T=4096, d=1024, I=512 on the
    persistent ones)."""
    cfg = synth.CONFIGS[cid] if cid == 2 else synth.CONFIGS[4].with_(name="prefill-zipf-bf16 T4096 d1024 I512",
                                                                     T=4096, d=1024, I=512)
    say(f"[stream] {cfg.name}: default stream, then a side stream")
    inp = synth.make_inputs(cfg)
    layer = layer_from_inputs(inp)
    x = upload(inp["x"])
    outs = []
    side = torch.cuda.Stream()
    for use_side in (False, True):
        b = upload(inp["bias"])
        for t in (layer.idx, layer.w, layer.counts, layer.row_src, layer.y_perm, layer.y, layer.ws):
            t.view(torch.uint8).fill_(0xFF)
        torch.cuda.synchronize()
        ctx = torch.cuda.stream(side) if use_side else torch.cuda.stream(torch.cuda.current_stream())
        with ctx:
            layer.forward(x, b)
            layer.update_bias(b, cfg.gamma)
            snap = dict(idx=layer.idx.clone(), w=layer.w.clone(), counts=layer.counts.clone(),
                        row_src=layer.row_src.clone(), y_perm=layer.y_perm.clone(), y=layer.y.clone(),
                        bias=b.clone())
        (side if use_side else torch.cuda.current_stream()).synchronize()
        outs.append(snap)
    torch.cuda.synchronize()
    for n in outs[0]:
        assert torch.equal(_bits(outs[0][n]), _bits(outs[1][n])), f"{cfg.name}: {n} differs on the side stream"
    say(f"[stream] {cfg.name}: side-stream run bit-identical")
