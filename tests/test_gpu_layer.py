"""GPU parity of the whole layer (route -> dispatch -> expert FFN -> combine ->
bias update) against the oracle's independent forward on the same seeded
inputs, per workload, up to the full-size prefill workloads bench.py times.

Tokens whose routing differs between the two sides must all be near-ties
(oracle fp64 gap < 1e-6); outputs are compared on the other tokens.  The
dispatch arrays and the bias step are compared bit-exactly against the
oracle fed the GPU's ids (conditional parity), and against the oracle's own
routing when no token flipped.  Every token goes through the oracle's
router; the routed FFN is checked on permuted rows at group and tile edges,
and the whole forward on sampled tokens (it is independent per token given
the bias)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from sparse_expert_routing_amd import _lib
from sparse_expert_routing_amd.layer import layer_from_inputs, upload
from tests.gpu_util import NEAR_TIE, TOL, bf16v, host, inputs_of, max_rel, say

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


def edge_rows(offsets, A, n_min, seed=0):
    """Permuted rows at every non-empty expert group's first and last row and
    at the 256-row tile edges inside each group (the last row of one tile and
    the first of the next), topped up with distinct random rows to at least
    min(n_min, A) rows (all A rows when n_min >= A)."""
    nz = np.where(np.diff(offsets) > 0)[0]
    parts = [offsets[nz], offsets[nz + 1] - 1]
    for e in nz:
        m = np.arange(offsets[e] + 256, offsets[e + 1], 256)
        parts += [m - 1, m]
    rows = np.unique(np.concatenate(parts))
    rows = rows[(rows >= 0) & (rows < A)]
    if len(rows) < n_min:
        rest = np.setdiff1d(np.arange(A), rows)
        rng = np.random.default_rng(seed)
        extra = rng.choice(rest, min(n_min - len(rows), len(rest)), replace=False)
        rows = np.unique(np.concatenate([rows, extra]))
    return rows.astype(np.int32)


def check_y_perm_rows(cfg, inp, layer, offsets, row_src, n_min):
    """y_perm on permuted rows at group and tile edges against the oracle's
    routed FFN fed the GPU's dispatch (its offsets and row order)."""
    A = cfg.T * cfg.k
    rows = edge_rows(offsets, A, n_min)
    tok = row_src // cfg.k
    if cfg.wt == "e4m3":
        q, s = oracle.quant_e4m3_rows(inp["x"])
        a_rows, a_sc = np.ascontiguousarray(q[tok]), np.ascontiguousarray(s[tok])
    else:
        a_rows, a_sc = np.ascontiguousarray(inp["x"][tok]), None
    say(f"[layer] {cfg.name}: oracle routed FFN on {len(rows)} permuted rows (group and tile edges)")
    yo = oracle.expert_ffn(oracle.shape_of(cfg), inp["experts"], offsets, a_rows, a_sc, rows=rows)
    del a_rows, a_sc
    yg = host(layer.y_perm[torch.from_numpy(rows).long().to(layer.y_perm.device)])
    if cfg.wt != "f32":
        yg, yo = bf16v(yg), bf16v(yo)
    err = max_rel(yg, yo)
    say(f"[layer] {cfg.name}: y_perm max rel err {err:.3e} on {len(rows)} rows")
    assert err <= TOL[cfg.wt], err


def check_layer(cfg, inp, n_sample, route_all=True, n_rows=0):
    """One forward + bias step on the GPU, compared with the oracle:
    - n_sample tokens end to end (ids, weights, y) through the oracle's own forward;
    - the dispatch arrays from the GPU's ids and the bias step from the GPU's
      counts, bit-exact (conditional parity: each stage fed its GPU upstream);
    - route_all: every token's ids (equal on each token that is not a
      near-tie), weights and gap through the oracle's router; when no token
      chooses differently, the dispatch arrays and the bias step also equal
      the oracle's own, bit for bit;
    - n_rows > 0: y_perm on at least n_rows permuted rows at group and tile
      edges."""
    say(f"[layer] {cfg.name}: upload + forward")
    layer = layer_from_inputs(inp)
    x = upload(inp["x"])
    b = upload(inp["bias"])
    y = layer.forward(x, b, gap=True)
    layer.update_bias(b, cfg.gamma)
    torch.cuda.synchronize()
    gi, gw, ggap = host(layer.idx), host(layer.w), host(layer.gap)
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
    gy = host(y[torch.from_numpy(toks).long().to(y.device)])
    err_y = max_rel(gy[ok], oy[ok])
    err_w = max_rel(gw[toks][ok], og[ok])
    say(f"[layer] {cfg.name}: sampled tokens: y max rel err {err_y:.3e}, weights {err_w:.3e}, near-ties "
        f"{int(near.sum())}, flipped {int(mism.sum())}")
    assert err_y <= TOL[cfg.wt], err_y
    assert err_w <= TOL["f32"], err_w

    # conditional parity of the dispatch and the bias step (bit-exact)
    cc, co, csrc, cof = oracle.dispatch(gi, cfg.E)
    assert np.array_equal(counts, cc) and np.array_equal(offsets, co), "counts/offsets differ"
    assert np.array_equal(row_src, csrc) and np.array_equal(row_of, cof), "permutation differs"
    cb = oracle.bias_update(inp["bias"], cc, cfg.k, cfg.T, cfg.gamma)
    assert np.array_equal(gb.view(np.uint32), cb.view(np.uint32)), "bias step differs"

    if route_all:
        say(f"[layer] {cfg.name}: oracle router on all {cfg.T} tokens")
        ri, rg, rgap, _ = oracle.route(sh, inp["x"], inp["wr"], inp["bias"])
        flip = np.any(gi != ri, axis=1)
        rnear = rgap < NEAR_TIE
        assert not np.any(flip & ~rnear), f"routing differs on non-near-tie tokens {np.where(flip & ~rnear)[0][:10]}"
        ok = ~flip
        err_w = max_rel(gw[ok], rg[ok])
        # the kernel's gap is the fp32 difference of two fp32 biased scores:
        # each score carries the fp32 logit accumulation error (~1e-6 x |logit|,
        # |logit| < 10 here) times sigmoid' <= 1/4, plus two fp32 roundings
        err_gap = float(np.abs(ggap[ok] - rgap[ok]).max())
        say(f"[layer] {cfg.name}: all tokens: near-ties {int(rnear.sum())}, flipped {int(flip.sum())}, "
            f"weights max rel err {err_w:.3e}, gap max abs err {err_gap:.2e}")
        assert err_w <= TOL["f32"], err_w
        assert err_gap <= 1e-5, err_gap
        if not flip.any():
            oc, oo, osrc, oof = oracle.dispatch(ri, cfg.E)
            assert np.array_equal(counts, oc) and np.array_equal(offsets, oo)
            assert np.array_equal(row_src, osrc) and np.array_equal(row_of, oof)
            ob = oracle.bias_update(inp["bias"], oc, cfg.k, cfg.T, cfg.gamma)
            assert np.array_equal(gb.view(np.uint32), ob.view(np.uint32))
    if n_rows:
        check_y_perm_rows(cfg, inp, layer, offsets, row_src, n_rows)
    return gi


def test_layer_config1_tiny_fp32_one_step():
    cfg = synth.CONFIGS[1]
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=cfg.T, n_rows=cfg.T * cfg.k)


def test_layer_config2_mid_bf16():
    cfg = synth.CONFIGS[2]
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=96, n_rows=512)


def test_layer_config2_ragged_T():
    cfg = synth.CONFIGS[2].with_(T=777)
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=48, n_rows=256)


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
    """The decode workload (T=64, d=7168, I=2048): every token routed through
    the oracle, y on sampled tokens, and y_perm on all 512 routed rows."""
    cfg = synth.CONFIGS[3]
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=24, n_rows=cfg.T * cfg.k)


def test_layer_config5_fp8_reduced():
    """The fp8 workload's recipe at a size the oracle finishes in seconds:
    T=600 (ragged), d=1024, I=256."""
    cfg = synth.CONFIGS[5].with_(T=600, d=1024, I=256)
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=64, n_rows=256)


def test_layer_config4_skewed_reduced():
    """The skewed workload's recipe (Zipf router rows, zero initial bias) at
    T=2048, d=1024, I=256: a few experts take most tokens (multi-tile groups)."""
    cfg = synth.CONFIGS[4].with_(T=2048, d=1024, I=256)
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=64, n_rows=512)


def test_layer_config4_full_size():
    """The skewed prefill workload at full size (T=16384, d=7168, I=2048, bf16),
    the launch configuration bench.py times: every token's ids, weights and
    gap through the oracle's router (ids equal off near-ties); the dispatch
    arrays and the bias step bit-exact; y_perm on at least 512 permuted rows
    at every group's first and last row and at the 256-row tile edges; y on
    12 sampled tokens through the oracle's whole forward."""
    cfg = synth.CONFIGS[4]
    inp = inputs_of(cfg)
    check_layer(cfg, inp, n_sample=12, n_rows=512)


def test_layer_config5_full_size():
    """The fp8 workload at full size (T=16384, d=7168, I=2048, e4m3 weights and
    activations): the persistent e4m3 GEMMs for the routed and shared
    experts; checked as the skewed prefill workload is."""
    cfg = synth.CONFIGS[5]
    inp = inputs_of(cfg)
    check_layer(cfg, inp, n_sample=12, n_rows=512)


def test_layer_past_32bit_offsets():
    """The whole layer at T=80000 tokens (d=7168, I=2048, bf16; 640000 routed
    rows, y_perm 4.6e9 elements): the routed GEMMs run on the small-tile
    kernels (the persistent ones address operands with 32-bit byte offsets),
    the shared expert and the combine on the persistent kernel; checked as
    the full-size workloads are (every token's routing, the dispatch arrays
    and the bias step bit-exact, y_perm at group and tile edges, sampled
    tokens end to end)."""
    cfg = synth.CONFIGS[4].with_(name="prefill-bf16 T80000 d7168 I2048", seed=28, T=80000, skew=0.0,
                                 bias="uniform")
    inp = synth.make_inputs(cfg)
    check_layer(cfg, inp, n_sample=8, n_rows=512)


def test_layer_ep8_shard_full_size():
    """One GPU's share of an 8-way expert-parallel layer at full size: the
    bias confines the choice to experts 0-31, so the grouped GEMMs run 32
    groups of about 4096 rows (T=16384, d=7168, I=2048, bf16); checked as the
    skewed prefill workload is."""
    cfg = synth.CONFIGS[6]
    inp = synth.make_inputs(cfg)
    gi = check_layer(cfg, inp, n_sample=12, n_rows=512)
    assert gi.max() < 32


def loop_parity(cfg, inp, steps, whole_layer):
    """Run `steps` steps of the balancing loop on the GPU (bias carried) and
    check each one stage by stage against the oracle fed the GPU's upstream
    values: the choice from the GPU's current bias (ids equal on every token
    that is not a near-tie), the counts from the GPU's ids and the new bias
    from the GPU's counts (both bit-exact).  The oracle's own loop, replayed
    independently, is compared too: bit-exact until the first near-tie token
    chooses differently.  The batch is fixed, so the oracle computes the
    fp64 affinities once.  whole_layer: every step is the whole forward
    (route, dispatch, routed FFN, shared expert + combine) and the bias step,
    as the benchmark runs it; otherwise route, dispatch and the bias step.
    Returns the max/mean load of every step."""
    T, k, E = cfg.T, cfg.k, cfg.E
    sh = oracle.shape_of(cfg)
    say(f"[loop] {cfg.name}: oracle affinities of all {T} tokens")
    _, _, _, s = oracle.route(sh, inp["x"], inp["wr"], inp["bias"], want_s=True)
    x, b = upload(inp["x"]), upload(inp["bias"])
    if whole_layer:
        layer = layer_from_inputs(inp)
        idx, counts = layer.idx, layer.counts
    else:
        ds = _lib.desc(T, cfg.d, E, k, cfg.I, cfg.act, cfg.wt)
        wr = upload(inp["wr"])
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
    say(f"[loop] {cfg.name}: {steps} steps ({'whole layer' if whole_layer else 'route, dispatch, bias step'})")
    for step in range(steps):
        if whole_layer:
            layer.step(x, b, gamma=cfg.gamma)
        else:
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
    say(f"[loop] {cfg.name}: {steps} steps stage-wise exact; near-tie tokens choosing differently: {flips}; "
        f"independent loops identical for {independent if independent is not None else steps} steps; "
        f"max/mean load {imb[0]:.2f} -> {imb[-1]:.2f}")
    return imb


def test_balancing_loop_reduced():
    """The bias-balancing loop (route -> counts -> sign-step update, 100 steps,
    bias carried) at the skewed workload's recipe, T=2048, d=1024, checked
    stage by stage at every step against the oracle (see loop_parity)."""
    cfg = synth.CONFIGS[4].with_(T=2048, d=1024, I=256)
    imb = loop_parity(cfg, synth.make_inputs(cfg), cfg.steps, whole_layer=False)
    assert imb[-1] < imb[0]


def test_balancing_loop_full_size():
    """The skewed prefill workload's balancing loop at full size (T=16384,
    d=7168, I=2048): 24 steps of the whole layer as bench.py runs them, each
    checked stage by stage against the oracle (see loop_parity)."""
    cfg = synth.CONFIGS[4]
    imb = loop_parity(cfg, inputs_of(cfg), 24, whole_layer=True)
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
