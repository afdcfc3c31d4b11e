"""GPU parity of the whole layer (route -> dispatch -> expert FFN -> combine ->
bias update) against the oracle's independent forward on the same seeded
inputs, per workload.

Tokens whose routing differs between the two sides must all be near-ties
(oracle fp64 gap < 1e-6); outputs are compared on the other tokens.  The
dispatch arrays and the bias step are compared bit-exactly when no token
flipped (when one did, the invariants are checked instead).  At the large
workloads the oracle computes sampled tokens one by one (the forward is
independent per token given the bias)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from sparse_expert_routing_amd import _lib
from sparse_expert_routing_amd.layer import layer_from_inputs, upload
from tests.gpu_util import NEAR_TIE, TOL, host, max_rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


def sample_tokens(T, n, seed=0):
    if n >= T:
        return np.arange(T, dtype=np.int32)
    rng = np.random.default_rng(seed)
    s = np.unique(np.concatenate([[0, T - 1], rng.choice(T, n - 2, replace=False)]))
    return s.astype(np.int32)


def check_layer(cfg, inp, n_sample, route_all=True):
    say(f"[layer] {cfg.name}: upload + forward")
    layer = layer_from_inputs(inp)
    x = upload(inp["x"])
    b = upload(inp["bias"])
    y = layer.forward(x, b, gap=True)
    layer.update_bias(b, cfg.gamma)
    torch.cuda.synchronize()
    gi, gw, gy = host(layer.idx), host(layer.w), host(y)
    counts, offsets, row_src, row_of = (host(t) for t in (layer.counts, layer.offsets, layer.row_src, layer.row_of))
    gb = host(b)
    sh = oracle.shape_of(cfg)

    toks = sample_tokens(cfg.T, n_sample)
    say(f"[layer] {cfg.name}: oracle forward on {len(toks)} tokens")
    oi, og, ogap, oy = oracle.forward(sh, inp["x"], inp["wr"], inp["bias"], inp["experts"], inp["shared"], toks)
    near = ogap < NEAR_TIE
    mism = np.any(gi[toks] != oi, axis=1)
    assert not np.any(mism & ~near), f"routing differs on non-near-tie tokens {toks[mism & ~near][:10]}"
    ok = ~mism
    err_y = max_rel(gy[toks][ok], oy[ok])
    err_w = max_rel(gw[toks][ok], og[ok])
    say(f"[layer] {cfg.name}: y max rel err {err_y:.3e}, weights {err_w:.3e}, sampled near-ties "
        f"{int(near.sum())}, flipped {int(mism.sum())}")
    assert err_y <= TOL[cfg.wt], err_y
    assert err_w <= TOL["f32"], err_w

    # invariants of the dispatch (no token dropped, a stable permutation)
    assert counts.sum() == cfg.T * cfg.k and offsets[-1] == cfg.T * cfg.k
    assert np.array_equal(row_of[row_src], np.arange(cfg.T * cfg.k))
    assert np.array_equal(np.bincount(gi.ravel(), minlength=256), counts)

    if route_all:
        ri, _, rgap, _ = oracle.route(sh, inp["x"], inp["wr"], inp["bias"])
        flip = np.any(gi != ri, axis=1)
        assert not np.any(flip & (rgap >= NEAR_TIE))
        say(f"[layer] {cfg.name}: all tokens: near-ties {int((rgap < NEAR_TIE).sum())}, flipped {int(flip.sum())}")
        if not flip.any():
            oc, oo, osrc, oof = oracle.dispatch(ri, 256)
            assert np.array_equal(counts, oc) and np.array_equal(offsets, oo)
            assert np.array_equal(row_src, osrc) and np.array_equal(row_of, oof)
            assert np.array_equal(gb, oracle.bias_update(inp["bias"], oc, cfg.k, cfg.T, cfg.gamma))
    return gi, gy


def test_layer_config1_tiny_fp32_one_step():
    cfg = synth.CONFIGS[1]
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=cfg.T)


def test_layer_config2_mid_bf16():
    cfg = synth.CONFIGS[2]
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=96)


def test_layer_config2_ragged_T():
    cfg = synth.CONFIGS[2].with_(T=777)
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=48)


@pytest.mark.parametrize("cid,over", [(1, {}), (2, {"T": 777}), (5, {"T": 600, "d": 1024, "I": 256}),
                                      (4, {"T": 2048, "d": 1024, "I": 256})])
def test_layer_gather_in_gemm_equals_materialised(cid, over):
    """The default forward (gate/up gathers through row_src) and the one over
    a materialised x_perm give the same y bit for bit."""
    cfg = synth.CONFIGS[cid].with_(**over) if over else synth.CONFIGS[cid]
    say(f"[layer] {cfg.name}: gathered vs materialised x_perm")
    inp = synth.make_inputs(cfg)
    layer = layer_from_inputs(inp)
    x, b = upload(inp["x"]), upload(inp["bias"])
    y1 = host(layer.forward(x, b, gather_in_gemm=True)).copy()
    y2 = host(layer.forward(x, b, gather_in_gemm=False))
    assert np.array_equal(y1, y2)


def test_layer_config3_decode_bf16():
    cfg = synth.CONFIGS[3]
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=24)


def test_layer_config5_fp8_reduced():
    """The fp8 workload's recipe at a size the oracle finishes in seconds:
    T=600 (ragged), d=1024, I=256."""
    cfg = synth.CONFIGS[5].with_(T=600, d=1024, I=256)
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=64)


def test_layer_config4_skewed_reduced():
    """The skewed workload's recipe (Zipf router rows, zero initial bias) at
    T=2048, d=1024, I=256: a few experts take most tokens (multi-tile groups)."""
    cfg = synth.CONFIGS[4].with_(T=2048, d=1024, I=256)
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=64)


def test_layer_config4_full_size_sampled():
    """The skewed prefill workload at full size (T=16384, d=7168, I=2048, bf16),
    the launch configuration bench.py times: the oracle checks 12 sampled
    tokens; every token's routing is checked for near-tie-only differences."""
    cfg = synth.CONFIGS[4]
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=12, route_all=False)


def test_layer_config5_full_size_sampled():
    """The fp8 workload at full size (T=16384, d=7168, I=2048, e4m3 weights and
    activations): the persistent fp8 GEMMs for the routed and shared experts;
    the oracle checks 12 sampled tokens."""
    cfg = synth.CONFIGS[5]
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=12, route_all=False)


def test_layer_ep8_shard_full_size_sampled():
    """One GPU's share of an 8-way expert-parallel layer at full size: the
    bias confines the choice to experts 0-31, so the grouped GEMMs run 32
    groups of about 4096 rows (T=16384, d=7168, I=2048, bf16); the oracle
    checks 12 sampled tokens."""
    cfg = synth.CONFIGS[6]
    inp = synth.make_inputs(cfg)
    gi, _ = check_layer(cfg, inp, n_sample=12, route_all=False)
    assert gi.max() < 32


def test_balancing_loop_reduced():
    """The bias-balancing loop (route -> counts -> sign-step update, 100 steps,
    bias carried) at the skewed workload's recipe, T=2048, d=1024, checked
    stage by stage at every step against the oracle fed the GPU's upstream
    values: the choice from the GPU's current bias (ids equal on every token
    that is not a near-tie), the counts from the GPU's ids and the new bias
    from the GPU's counts (both bit-exact).  The oracle's own loop, replayed
    independently, is compared too: bit-exact until the first near-tie token
    chooses differently.  The batch is fixed, so the oracle computes the fp64
    affinities once."""
    cfg = synth.CONFIGS[4].with_(T=2048, d=1024, I=256)
    T, k, E = cfg.T, cfg.k, cfg.E
    inp = synth.make_inputs(cfg)
    sh = oracle.shape_of(cfg)
    _, _, _, s = oracle.route(sh, inp["x"], inp["wr"], inp["bias"], want_s=True)
    ds = _lib.desc(T, cfg.d, E, k, cfg.I, cfg.act, cfg.wt)
    x, wr, b = upload(inp["x"]), upload(inp["wr"]), upload(inp["bias"])
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    row_src = torch.empty(T * k, dtype=torch.int32, device="cuda")
    row_of = torch.empty(T * k, dtype=torch.int32, device="cuda")
    nws = max(_lib.workspace_bytes(ds, st) for st in (_lib.MOE_WS_DISPATCH, _lib.MOE_WS_ROUTE))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    gb_prev = np.array(inp["bias"], dtype=np.float32)
    ob = gb_prev.copy()  # the oracle's own loop
    independent = None
    flips = 0
    imb = []
    for step in range(cfg.steps):
        _lib.moe_route(ds, x, wr, b, idx, w, None, ws)
        _lib.moe_dispatch(ds, idx, None, counts, offsets, row_src, row_of, None, None, ws)
        _lib.moe_bias_update(ds, counts, cfg.gamma, b)
        torch.cuda.synchronize()
        gi, gc, gb = host(idx), host(counts), host(b)
        # conditional parity: each stage from the GPU's upstream values
        ci, _, cgap = oracle.choose(s, gb_prev, k)
        flip = np.any(gi != ci, axis=1)
        assert not np.any(flip & (cgap >= NEAR_TIE)), f"step {step}: a non-near-tie token chose differently"
        flips += int(flip.sum())
        oc, _, _, _ = oracle.dispatch(gi, E)
        assert np.array_equal(gc, oc), f"step {step}: counts differ"
        nb = oracle.bias_update(gb_prev, gc, k, T, cfg.gamma)
        assert np.array_equal(gb.view(np.uint32), nb.view(np.uint32)), f"step {step}: bias differs"
        imb.append(gc.max() / gc.mean())
        # the oracle's independent loop
        if independent is None:
            oi, _, _ = oracle.choose(s, ob, k)
            if np.array_equal(oi, gi):
                ob = oracle.bias_update(ob, oracle.dispatch(oi, E)[0], k, T, cfg.gamma)
            else:
                independent = step
        gb_prev = gb
    say(f"[loop] {cfg.steps} steps stage-wise exact; near-tie tokens choosing differently: {flips}; "
        f"independent loops identical for {independent if independent is not None else cfg.steps} steps; "
        f"max/mean load {imb[0]:.2f} -> {imb[-1]:.2f}")
    assert imb[-1] < imb[0]


def test_balancing_loop_fresh_batches_and_gamma_switch():
    """The balancing loop as training runs it: a fresh batch every step
    (skewed workload's recipe, T=2048, d=1024), and the bias step size from
    the schedule (0.001, then 0 once 14.3T tokens have been consumed: the
    loop starts 16 steps before that point).  Each step is checked against
    the oracle fed the GPU's current bias and that step's batch: ids equal on
    every token that is not a near-tie, counts and the new bias bit-exact;
    after the switch the bias stays bit-for-bit constant while routing
    goes on."""
    from sparse_expert_routing_amd.layer import GAMMA, GAMMA_TOKENS, bias_gamma
    cfg = synth.CONFIGS[4].with_(T=2048, d=1024, I=256)
    T, k, E = cfg.T, cfg.k, cfg.E
    steps, switch = 24, 16
    inp = synth.make_inputs(cfg)
    sh = oracle.shape_of(cfg)
    ds = _lib.desc(T, cfg.d, E, k, cfg.I, cfg.act, cfg.wt)
    wr, b = upload(inp["wr"]), upload(inp["bias"])
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    row_src = torch.empty(T * k, dtype=torch.int32, device="cuda")
    row_of = torch.empty(T * k, dtype=torch.int32, device="cuda")
    nws = max(_lib.workspace_bytes(ds, st) for st in (_lib.MOE_WS_DISPATCH, _lib.MOE_WS_ROUTE))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    gb_prev = np.array(inp["bias"], dtype=np.float32)
    flips = 0
    imb = []
    for step in range(steps):
        tokens_seen = GAMMA_TOKENS - (switch - step) * T
        gamma = bias_gamma(tokens_seen)
        assert gamma == (GAMMA if step < switch else 0.0)
        xs = synth.make_x_step(cfg, step)
        _lib.moe_route(ds, upload(xs), wr, b, idx, w, None, ws)
        _lib.moe_dispatch(ds, idx, None, counts, offsets, row_src, row_of, None, None, ws)
        _lib.moe_bias_update(ds, counts, gamma, b)
        torch.cuda.synchronize()
        gi, gc, gb = host(idx), host(counts), host(b)
        oi, _, ogap, _ = oracle.route(sh, xs, inp["wr"], gb_prev)
        flip = np.any(gi != oi, axis=1)
        assert not np.any(flip & (ogap >= NEAR_TIE)), f"step {step}: a non-near-tie token chose differently"
        flips += int(flip.sum())
        assert np.array_equal(gc, oracle.dispatch(gi, E)[0]), f"step {step}: counts differ"
        nb = oracle.bias_update(gb_prev, gc, k, T, gamma)
        assert np.array_equal(gb.view(np.uint32), nb.view(np.uint32)), f"step {step}: bias differs"
        if step >= switch:
            assert np.array_equal(gb.view(np.uint32), gb_prev.view(np.uint32)), f"step {step}: bias moved at gamma 0"
        imb.append(gc.max() / gc.mean())
        gb_prev = gb
    say(f"[loop] fresh batches: {steps} steps stage-wise exact, gamma 0 from step {switch}; "
        f"near-tie tokens choosing differently: {flips}; max/mean load {imb[0]:.2f} -> {imb[switch - 1]:.2f}")
    assert imb[switch - 1] < imb[0]
