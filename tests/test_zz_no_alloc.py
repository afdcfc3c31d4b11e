"""moe_dispatch_noalloc (the dispatch for callers that cannot allocate: its
block-count table lives in the library's static device scratch) against
moe_dispatch with a caller workspace, through the C ABI: every output bit for
bit, on two calls in a row, the second with fewer tokens (the scratch keeps
the first call's contents), for the bf16 row copy, the e4m3 quantising
gather and the bookkeeping-only form."""
import numpy as np
import pytest
import torch

import synth
from sparse_expert_routing_amd import _lib
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


def _outputs(T, d, wt, gather):
    i32 = dict(dtype=torch.int32, device="cuda")
    o = dict(counts=torch.full((256,), -7, **i32), offsets=torch.full((257,), -7, **i32),
             row_src=torch.full((T * 8,), -7, **i32), row_of=torch.full((T * 8,), -7, **i32),
             x_perm=None, x_perm_scale=None)
    if gather:
        o["x_perm"] = torch.full((T * 8, d), 0x55, dtype=torch.uint8 if wt == "e4m3" else torch.int16, device="cuda")
        if wt == "e4m3":
            o["x_perm_scale"] = torch.full((T * 8, d // 128), 0x55, dtype=torch.uint8, device="cuda")
    return o


@pytest.mark.parametrize("wt,gather", [("bf16", True), ("e4m3", True), ("bf16", False)])
def test_dispatch_noalloc_matches_dispatch(wt, gather):
    d = 1024
    for call, T in enumerate((5000, 777)):  # the second call is smaller
        say(f"[noalloc] call {call}: T={T} wt={wt} gather={gather}")
        cfg = synth.Config("noalloc", seed=31 + call, T=T, d=d, I=256, wt=wt)
        ids = np.sort(synth.random_ids(cfg.seed, synth.TID_IDS, T, 256, 8), axis=1)
        x = synth.normal(cfg.seed, synth.TID_X, (T, d), 1.0, "bf16")
        ds = _lib.desc(T, d, 256, 8, 256, "bf16", wt)
        idx_d, x_d = dev(ids), dev(x)
        ref, got = _outputs(T, d, wt, gather), _outputs(T, d, wt, gather)
        ws = torch.empty(_lib.workspace_bytes(ds, _lib.MOE_WS_DISPATCH), dtype=torch.uint8, device="cuda")
        _lib.moe_dispatch(ds, idx_d, x_d, ref["counts"], ref["offsets"], ref["row_src"], ref["row_of"],
                          ref["x_perm"], ref["x_perm_scale"], ws)
        _lib.moe_dispatch_noalloc(ds, idx_d, x_d, got["counts"], got["offsets"], got["row_src"], got["row_of"],
                                  got["x_perm"], got["x_perm_scale"])
        torch.cuda.synchronize()
        for n, t in ref.items():
            if t is not None:
                assert torch.equal(t, got[n]), f"call {call} (T={T}): {n} differs"
        assert int(ref["offsets"][-1]) == T * 8


def test_dispatch_noalloc_rejects_too_many_tokens():
    T = (1 << 20) + 1
    ds = _lib.desc(T, 1024, 256, 8, 256, "bf16", "bf16")
    p = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(_lib.MoeError) as ei:
        _lib.moe_dispatch_noalloc(ds, p, p, p, p, p, p, None, None)
    assert ei.value.status == _lib.MOE_ESCRATCH
