"""GPU parity, stage by stage: each C-ABI call against the oracle function of the
same stage, on the same seeded inputs (none of them produced by the HIP path).

Bars: integer and byte outputs bit-exact; routing ids bit-exact except on
near-tie tokens (oracle fp64 gap between the 8th and 9th biased score below
1e-6), which are counted and reported; floating outputs within the max
relative error ||a - r||_inf / ||r||_inf of 1e-4 (fp32), 2e-2 (bf16),
5e-2 (e4m3)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import sparse_expert_routing_amd as moe
from sparse_expert_routing_amd import _lib
from tests.gpu_util import NEAR_TIE, TOL, bf16v, dev, empty, host, max_rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()


# ------------------------------------------------------------------ route

def run_route(cfg, x, wr, bias):
    ds = _lib.desc(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, cfg.act, cfg.wt)
    idx = empty((cfg.T, cfg.k), torch.int32)
    w = empty((cfg.T, cfg.k), torch.float32)
    gap = empty(cfg.T, torch.float32)
    ws = empty(max(_lib.workspace_bytes(ds, _lib.MOE_WS_ROUTE), 256), torch.uint8)
    moe.moe_route(ds, dev(x), dev(wr), dev(bias), idx, w, gap, ws)
    torch.cuda.synchronize()
    return host(idx), host(w), host(gap)


def check_route(cfg, x, wr, bias, label):
    say(f"[route] {label} T={cfg.T} d={cfg.d} act={cfg.act}")
    gi, gw, ggap = run_route(cfg, x, wr, bias)
    oi, og, ogap, _ = oracle.route(oracle.shape_of(cfg), x, wr, bias)
    near = ogap < NEAR_TIE
    mism = np.any(gi != oi, axis=1)
    say(f"[route] {label}: near-ties {int(near.sum())}, flipped {int(mism.sum())} of {cfg.T} tokens")
    assert not np.any(mism & ~near), f"ids differ on non-near-tie tokens {np.where(mism & ~near)[0][:10]}"
    ok = ~mism
    assert np.all(np.diff(gi, axis=1) > 0)  # ascending, distinct
    err = max_rel(gw[ok], og[ok])
    assert err <= TOL["f32"], err
    np.testing.assert_allclose(gw.astype(np.float64).sum(axis=1), 1.0, atol=1e-5)
    assert np.abs(ggap[ok] - ogap[ok]).max() < 1e-5
    return gi, near, mism


@pytest.mark.parametrize("cid,T", [(1, None), (2, 300), (2, None), (3, None), (2, 1)])
def test_route_configs(cid, T):
    cfg = synth.CONFIGS[cid]
    if T is not None:
        cfg = cfg.with_(T=T)
    x, wr, bias = synth.make_router(cfg)
    check_route(cfg, x, wr, bias, f"config {cid}")


@pytest.mark.parametrize("T,d", [(100, 896), (100, 1408), (129, 7168)])
def test_route_uneven_k_splits(T, d):
    # small T splits the router's K range over several workgroups; these d
    # give splits of unequal length and fold points inside a split
    cfg = synth.CONFIGS[2].with_(T=T, d=d)
    x, wr, bias = synth.make_router(cfg)
    check_route(cfg, x, wr, bias, f"T={T} d={d}")


def test_route_zero_router_ties_go_to_lower_ids():
    cfg = synth.CONFIGS[2].with_(T=130, d=512)
    x, _, _ = synth.make_router(cfg)
    wr = np.zeros((256, cfg.d), np.float32)
    gi, gw, ggap = run_route(cfg, x, wr, np.zeros(256, np.float32))
    assert np.array_equal(gi, np.tile(np.arange(8), (cfg.T, 1)))
    assert np.all(gw == np.float32(0.125)) and np.all(ggap == 0)


def test_route_huge_bias_forces_the_same_experts():
    cfg = synth.CONFIGS[2].with_(T=200, d=512)
    x, wr, _ = synth.make_router(cfg)
    bias = np.zeros(256, np.float32)
    hot = [3, 17, 64, 65, 128, 200, 254, 255]
    bias[hot] = 10.0
    gi, gw, _ = run_route(cfg, x, wr, bias)
    assert np.all(gi == np.array(hot))
    oi, og, _, _ = oracle.route(oracle.shape_of(cfg), x, wr, bias)
    assert np.array_equal(gi, oi) and max_rel(gw, og) <= TOL["f32"]


# --------------------------------------------------------------- dispatch

def run_dispatch(T, d, act, wt, idx, x):
    ds = _lib.desc(T, d, 256, 8, 128, act, wt)
    A = T * 8
    counts, offsets = empty(256, torch.int32), empty(257, torch.int32)
    row_src, row_of = empty(A, torch.int32), empty(A, torch.int32)
    gin = {"f32": torch.float32, "bf16": torch.int16, "e4m3": torch.uint8}[wt]
    x_perm = empty((A, d), gin)
    xs = empty((A, d // 128), torch.uint8) if wt == "e4m3" else None
    ws = empty(_lib.workspace_bytes(ds, _lib.MOE_WS_DISPATCH), torch.uint8)
    moe.moe_dispatch(ds, dev(idx), dev(x), counts, offsets, row_src, row_of, x_perm, xs, ws)
    torch.cuda.synchronize()
    return [host(t) for t in (counts, offsets, row_src, row_of, x_perm)] + [host(xs) if xs is not None else None]


def ids_case(kind, T):
    if kind == "random":
        return synth.random_ids(T, synth.TID_IDS, T, 256, 8)
    if kind == "same8":
        return np.tile(np.array([0, 5, 9, 100, 101, 200, 250, 255], np.int32), (T, 1))
    # skewed: every token takes experts 0, 1, 2 plus 5 random others
    tail = synth.random_ids(T + 1, synth.TID_IDS, T, 253, 5) + 3
    return np.ascontiguousarray(np.concatenate([np.tile(np.arange(3, dtype=np.int32), (T, 1)), tail], axis=1))


# random routings at every size; the degenerate ones (all tokens on the same
# 8 experts, three hot experts) at two sizes
DISPATCH_CASES = [(kind, T) for kind in ("random", "same8", "skewed")
                  for T in ((1, 255, 256, 257, 1000, 4096) if kind == "random" else (257, 1000))]


@pytest.mark.parametrize("kind,T", DISPATCH_CASES)
@pytest.mark.parametrize("act,wt,d", [("f32", "f32", 256), ("bf16", "bf16", 512), ("bf16", "e4m3", 384)])
def test_dispatch_bit_exact(T, act, wt, d, kind):
    say(f"[dispatch] T={T} d={d} {act}/{wt} {kind}")
    idx = ids_case(kind, T)
    x = synth.normal(7, synth.TID_X, (T, d), 1.0, act)
    if T > 3:
        x[3] = 0  # an all-zero row: e4m3 scale 1, codes 0
    counts, offsets, row_src, row_of, x_perm, xs = run_dispatch(T, d, act, wt, idx, x)
    oc, oo, osrc, oof = oracle.dispatch(idx, 256)
    assert np.array_equal(counts, oc) and np.array_equal(offsets, oo)
    assert np.array_equal(row_src, osrc) and np.array_equal(row_of, oof)
    tok = osrc // 8
    if wt == "e4m3":
        q, s = oracle.quant_e4m3_rows(x, act)
        assert np.array_equal(x_perm, q[tok]) and np.array_equal(xs, s[tok])
    else:
        assert np.array_equal(x_perm, x[tok])


def test_dispatch_out_of_range_ids_are_not_dispatched():
    """Ids outside [0, E) (a precondition violation) stay in bounds: they take
    no row, their row_of entry is -1 and offsets[E] falls short of T*k by
    their number; the valid assignments are grouped as usual (the stable
    order of numpy's argsort over the valid flat assignments)."""
    T, d = 600, 256
    say(f"[dispatch] T={T}: out-of-range ids")
    idx = synth.random_ids(5, synth.TID_IDS, T, 256, 8)
    idx[::7, 3] = -1
    idx[::11, 6] = 256
    idx[5, 0] = 1 << 30
    x = synth.normal(7, synth.TID_X, (T, d), 1.0, "bf16")
    counts, offsets, row_src, row_of, x_perm, _ = run_dispatch(T, d, "bf16", "bf16", idx, x)
    flat = idx.ravel()
    valid = (flat >= 0) & (flat < 256)
    nv = int(valid.sum())
    assert nv < T * 8
    assert np.array_equal(counts, np.bincount(flat[valid], minlength=256))
    assert offsets[-1] == nv and np.array_equal(offsets[:-1], np.concatenate([[0], np.cumsum(counts)[:-1]]))
    fv = np.where(valid)[0]
    order = fv[np.argsort(flat[fv], kind="stable")]
    assert np.array_equal(row_src[:nv], order)
    assert np.all(row_of[~valid] == -1) and np.array_equal(row_of[order], np.arange(nv))
    assert np.array_equal(x_perm[:nv], x[order // 8])


# ------------------------------------------------------------- expert FFN

def run_ffn(cfg, offsets, a_rows, a_scales, experts):
    ds = _lib.desc(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, cfg.act, cfg.wt)
    A = cfg.T * cfg.k
    w = {n: (dev(a) if a is not None else None) for n, a in experts.items()}
    fw = _lib.ffn_weights(w["gate"], w["up"], w["down"], w["s_gate"], w["s_up"], w["s_down"])
    y = empty((A, cfg.d), torch.float32 if cfg.wt == "f32" else torch.int16)
    ws = empty(_lib.workspace_bytes(ds, _lib.MOE_WS_FFN), torch.uint8)
    moe.moe_expert_ffn(ds, dev(a_rows), dev(a_scales) if a_scales is not None else None, dev(offsets), fw, y, ws)
    torch.cuda.synchronize()
    return host(y)


def ffn_inputs(cfg, kind):
    x = synth.normal(cfg.seed, synth.TID_X, (cfg.T, cfg.d), 1.0, cfg.act)
    idx = ids_case(kind, cfg.T)
    _, offsets, row_src, _ = oracle.dispatch(idx, 256)
    tok = row_src // 8
    if cfg.wt == "e4m3":
        q, s = oracle.quant_e4m3_rows(x, cfg.act)
        return offsets, np.ascontiguousarray(q[tok]), np.ascontiguousarray(s[tok])
    return offsets, np.ascontiguousarray(x[tok]), None


def yvals(y, wt):
    return y.astype(np.float64) if wt == "f32" else bf16v(y).astype(np.float64)


@pytest.mark.parametrize("wt", ["f32", "bf16", "e4m3"])
@pytest.mark.parametrize("kind,T", [("random", 40), ("same8", 300), ("skewed", 257)])
def test_expert_ffn_small(wt, kind, T):
    act = "f32" if wt == "f32" else "bf16"
    cfg = synth.Config("ffn", seed=21, T=T, d=256, I=128, act=act, wt=wt)
    say(f"[ffn] {wt} {kind} T={T}")
    experts = synth.make_ffn(cfg, 256, (synth.TID_GATE, synth.TID_UP, synth.TID_DOWN))
    offsets, a_rows, a_sc = ffn_inputs(cfg, kind)
    y = run_ffn(cfg, offsets, a_rows, a_sc, experts)
    yo = oracle.expert_ffn(oracle.shape_of(cfg), experts, offsets, a_rows, a_sc)
    err = max_rel(yvals(y, wt), yvals(yo, wt))
    say(f"[ffn] {wt} {kind} T={T}: max rel err {err:.3e}")
    assert err <= TOL[wt], err


@pytest.mark.parametrize("T,d,I", [(257, 256, 128), (4096, 512, 256)])
def test_expert_ffn_e4m3_arbitrary_scale_bytes(T, d, I):
    """Every e4m3 scale crosses the interface as an E8M0 byte (2^(e - 127)),
    so a scale is a power of two by construction.  Here the weight block
    scales and the activation tile scales are not the quantiser's: random
    bytes over 2^-12 .. 2^12 (block by block and tile by tile), which the
    block-scaled MFMAs must apply exactly as the oracle's E8M0 decoder reads
    them (small-tile kernel at T=257, the persistent kernel at T=4096)."""
    cfg = synth.Config("ffn-e8m0", seed=27, T=T, d=d, I=I, wt="e4m3")
    say(f"[ffn] e4m3 arbitrary scale bytes T={T} d={d} I={I}")
    experts = synth.make_ffn(cfg, 256, (synth.TID_GATE, synth.TID_UP, synth.TID_DOWN))
    rng = np.random.default_rng(T)
    for n in ("s_gate", "s_up", "s_down"):
        experts[n] = rng.integers(127 - 12, 127 + 13, experts[n].shape).astype(np.uint8)
    offsets, a_rows, a_sc = ffn_inputs(cfg, "random")
    a_sc = rng.integers(127 - 12, 127 + 13, a_sc.shape).astype(np.uint8)
    y = run_ffn(cfg, offsets, a_rows, a_sc, experts)
    rows = None if T <= 257 else np.unique(rng.integers(0, cfg.A, 256)).astype(np.int32)
    yo = oracle.expert_ffn(oracle.shape_of(cfg), experts, offsets, a_rows, a_sc, rows=rows)
    yg = y if rows is None else y[rows]
    err = max_rel(yvals(yg, "e4m3"), yvals(yo, "e4m3"))
    say(f"[ffn] e4m3 arbitrary scale bytes T={T}: max rel err {err:.3e}")
    assert err <= TOL["e4m3"], err


@pytest.mark.parametrize("T,d,I", [(40, 256, 128), (4096, 512, 256)])
def test_expert_ffn_e4m3_nan_scale_byte(T, d, I):
    """E8M0 byte 255 is the format's NaN, not a scale: a weight block given it
    makes exactly the outputs that block feeds NaN (the down block (0, 0) of
    the largest group: that expert's rows x output columns 0..127) and
    leaves every other output finite (small-tile and persistent kernels)."""
    cfg = synth.Config("ffn-nan", seed=21, T=T, d=d, I=I, wt="e4m3")
    say(f"[ffn] e4m3 NaN scale byte T={T} d={d} I={I}")
    experts = synth.make_ffn(cfg, 256, (synth.TID_GATE, synth.TID_UP, synth.TID_DOWN))
    offsets, a_rows, a_sc = ffn_inputs(cfg, "random")
    e = int(np.argmax(np.diff(offsets)))
    experts["s_down"][e, 0, 0] = 255
    yv = yvals(run_ffn(cfg, offsets, a_rows, a_sc, experts), "e4m3")
    rows = np.zeros(cfg.A, bool)
    rows[offsets[e]:offsets[e + 1]] = True
    assert np.isnan(yv[rows, :128]).all()
    assert np.isfinite(yv[rows, 128:]).all() and np.isfinite(yv[~rows]).all()


@pytest.mark.parametrize("kind,T,d,I", [("random", 40, 1024, 512), ("skewed", 100, 512, 512), ("same8", 17, 512, 1024),
                                      ("random", 1, 512, 512), ("same8", 16, 1536, 512), ("random", 128, 512, 512)])
def test_expert_ffn_tiny_groups(kind, T, d, I):
    """Decode-sized groups (T*8 <= 4*256 rows, bf16): the weight-streaming
    path with K split over the waves and 16-row passes.  Cases: empty
    experts, a single row, exactly 16 rows, 17 rows (a second pass of one
    row), 100-row hot experts (seven passes), a chunk count per wave that is
    not a power of two (d=1536: 6), and the largest T the path takes."""
    cfg = synth.Config("ffn-tiny", seed=22, T=T, d=d, I=I, wt="bf16")
    say(f"[ffn] tiny groups {kind} T={T} d={d} I={I}")
    experts = synth.make_ffn(cfg, 256, (synth.TID_GATE, synth.TID_UP, synth.TID_DOWN))
    offsets, a_rows, a_sc = ffn_inputs(cfg, kind)
    y = run_ffn(cfg, offsets, a_rows, a_sc, experts)
    yo = oracle.expert_ffn(oracle.shape_of(cfg), experts, offsets, a_rows, a_sc)
    err = max_rel(yvals(y, "bf16"), yvals(yo, "bf16"))
    say(f"[ffn] tiny groups {kind} T={T}: max rel err {err:.3e}")
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("wt", ["bf16", "e4m3"])
@pytest.mark.parametrize("kind", ["random", "skewed", "same8"])
def test_expert_ffn_large_groups(kind, wt):
    """T=4096 tokens: 128+ rows per expert on average, the persistent
    256x256-tile path (bf16, and e4m3 with its fp32 promotion per 128 of K
    and the fused h quantisation); d=512, I=256 so several column tiles and
    K stages run.  The oracle checks 160 sampled permuted rows including
    group edges."""
    cfg = synth.Config("ffn-large", seed=23, T=4096, d=512, I=256, wt=wt)
    say(f"[ffn] large groups {wt} {kind}")
    experts = synth.make_ffn(cfg, 256, (synth.TID_GATE, synth.TID_UP, synth.TID_DOWN))
    offsets, a_rows, a_sc = ffn_inputs(cfg, kind)
    y = run_ffn(cfg, offsets, a_rows, a_sc, experts)
    rng = np.random.default_rng(1)
    nz = np.where(np.diff(offsets) > 0)[0]
    edges = np.concatenate([offsets[nz], offsets[nz + 1] - 1, offsets[nz] + 255, offsets[nz] + 256])
    edges = edges[edges < cfg.A]
    rows = np.unique(np.concatenate([rng.choice(edges, min(96, len(edges)), replace=False),
                                     rng.integers(0, cfg.A, 64)])).astype(np.int32)
    yo = oracle.expert_ffn(oracle.shape_of(cfg), experts, offsets, a_rows, a_sc, rows=rows)
    err = max_rel(yvals(y[rows], wt), yvals(yo, wt))
    say(f"[ffn] large groups {wt} {kind}: max rel err {err:.3e} on {len(rows)} rows")
    assert err <= TOL[wt], err


@pytest.mark.parametrize("wt", ["bf16", "e4m3"])
def test_expert_ffn_past_32bit_offsets(wt):
    """The largest operands: T=80000 tokens at the prefill shape (d=7168,
    I=2048), 640000 routed rows.  x_perm then holds 4.6e9 elements, past the
    32-bit byte offsets of the persistent kernels (the host routes the
    routed FFN to the small-tile kernels) and past 2^32 elements, so the
    small-tile kernels' row offsets must be 64-bit.  The oracle checks the
    rows at every group edge, the last row and random rows."""
    T, d, I = 80000, 7168, 2048
    cfg = synth.Config("ffn-huge", seed=27, T=T, d=d, I=I, wt=wt)
    say(f"[ffn] past 32-bit offsets {wt} T={T} d={d} I={I}: generating inputs")
    experts = synth.make_ffn(cfg, 256, (synth.TID_GATE, synth.TID_UP, synth.TID_DOWN))
    offsets, a_rows, a_sc = ffn_inputs(cfg, "random")
    assert cfg.A * d >= (1 << 32)
    say(f"[ffn] past 32-bit offsets {wt}: GPU")
    y = run_ffn(cfg, offsets, a_rows, a_sc, experts)
    rng = np.random.default_rng(2)
    nz = np.where(np.diff(offsets) > 0)[0]
    edges = np.concatenate([offsets[nz], offsets[nz + 1] - 1, [cfg.A - 1]])
    rows = np.unique(np.concatenate([edges, rng.integers(0, cfg.A, 32)])).astype(np.int32)
    assert int(rows.max()) * d >= (1 << 32)
    say(f"[ffn] past 32-bit offsets {wt}: oracle on {len(rows)} rows")
    yo = oracle.expert_ffn(oracle.shape_of(cfg), experts, offsets, a_rows, a_sc, rows=rows)
    err = max_rel(yvals(y[rows], wt), yvals(yo, wt))
    say(f"[ffn] past 32-bit offsets {wt}: max rel err {err:.3e} on {len(rows)} rows")
    assert err <= TOL[wt], err


def test_expert_ffn_config2_sampled_rows():
    """Config 2 shapes (T=2048, d=2048, I=512), bf16, real routing; the oracle
    checks 64 sampled permuted rows, including each group's first and last."""
    cfg = synth.CONFIGS[2]
    say("[ffn] config 2 sampled rows")
    inp = synth.make_inputs(cfg)
    idx, _, _, _ = oracle.route(oracle.shape_of(cfg), inp["x"], inp["wr"], inp["bias"])
    _, offsets, row_src, _ = oracle.dispatch(idx, 256)
    a_rows = np.ascontiguousarray(inp["x"][row_src // 8])
    y = run_ffn(cfg, offsets, a_rows, None, inp["experts"])
    rng = np.random.default_rng(0)
    nz = np.where(np.diff(offsets) > 0)[0]
    rows = np.unique(np.concatenate([offsets[nz], offsets[nz + 1] - 1, rng.integers(0, cfg.A, 32)]))[:64]
    yo = oracle.expert_ffn(oracle.shape_of(cfg), inp["experts"], offsets, a_rows, None, rows=rows)
    err = max_rel(yvals(y[rows], "bf16"), yvals(yo, "bf16"))
    say(f"[ffn] config 2: max rel err {err:.3e} on {len(rows)} rows")
    assert err <= TOL["bf16"], err


# ------------------------------------- the dispatch gather folded into the GEMM

@pytest.mark.parametrize("T", [1, 257, 4096])
def test_dispatch_bookkeeping_only(T):
    """x_perm = NULL: counts, offsets, row_src, row_of as the oracle's, nothing gathered."""
    say(f"[dispatch] bookkeeping only T={T}")
    ds = _lib.desc(T, 512, 256, 8, 128, "bf16", "bf16")
    idx = ids_case("random", T)
    counts, offsets = empty(256, torch.int32), empty(257, torch.int32)
    row_src, row_of = empty(T * 8, torch.int32), empty(T * 8, torch.int32)
    ws = empty(_lib.workspace_bytes(ds, _lib.MOE_WS_DISPATCH), torch.uint8)
    moe.moe_dispatch(ds, dev(idx), None, counts, offsets, row_src, row_of, None, None, ws)
    torch.cuda.synchronize()
    oc, oo, osrc, oof = oracle.dispatch(idx, 256)
    assert np.array_equal(host(counts), oc) and np.array_equal(host(offsets), oo)
    assert np.array_equal(host(row_src), osrc) and np.array_equal(host(row_of), oof)


def run_ffn_rows(cfg, offsets, row_src, x, experts):
    ds = _lib.desc(cfg.T, cfg.d, cfg.E, cfg.k, cfg.I, cfg.act, cfg.wt)
    w = {n: (dev(a) if a is not None else None) for n, a in experts.items()}
    fw = _lib.ffn_weights(w["gate"], w["up"], w["down"], w["s_gate"], w["s_up"], w["s_down"])
    y = empty((cfg.T * cfg.k, cfg.d), torch.float32 if cfg.wt == "f32" else torch.int16)
    ws = empty(_lib.workspace_bytes(ds, _lib.MOE_WS_FFN), torch.uint8)
    moe.moe_expert_gate_up_rows(ds, dev(x), dev(row_src), dev(offsets), fw, ws)
    moe.moe_expert_down(ds, dev(offsets), fw, y, ws)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("wt,T,d,I,kind", [("f32", 40, 256, 128, "random"), ("bf16", 300, 256, 128, "same8"),
                                           ("bf16", 4096, 512, 256, "skewed"), ("bf16", 100, 512, 512, "skewed"),
                                           ("e4m3", 257, 256, 128, "skewed"),
                                           ("e4m3", 1000, 256, 128, "random"),
                                           ("e4m3", 4096, 512, 256, "skewed"), ("e4m3", 4097, 512, 256, "random")])
def test_gate_up_rows_matches_materialised(wt, T, d, I, kind):
    """Gate/up reading the token rows through row_src (no x_perm) gives the
    same y_perm bit for bit as the GEMM over the materialised x_perm (same
    rows, same order, same kernels); small-group, large-group (T=4096) and
    e4m3 (x quantised once per token, its tile scales laid out per 128-block
    in GEMM row order for the persistent kernel at T >= 4096) paths.  Parity
    of this path with the oracle is the layer tests' (the layer uses it by
    default)."""
    act = "f32" if wt == "f32" else "bf16"
    cfg = synth.Config("ffn-rows", seed=25, T=T, d=d, I=I, act=act, wt=wt)
    say(f"[ffn] gathered gate/up {wt} T={T} d={d} I={I} {kind}")
    experts = synth.make_ffn(cfg, 256, (synth.TID_GATE, synth.TID_UP, synth.TID_DOWN))
    x = synth.normal(cfg.seed, synth.TID_X, (T, d), 1.0, act)
    _, offsets, row_src, _ = oracle.dispatch(ids_case(kind, T), 256)
    tok = row_src // 8
    if wt == "e4m3":
        q, s = oracle.quant_e4m3_rows(x, act)
        a_rows, a_sc = np.ascontiguousarray(q[tok]), np.ascontiguousarray(s[tok])
    else:
        a_rows, a_sc = np.ascontiguousarray(x[tok]), None
    y_mat = run_ffn(cfg, offsets, a_rows, a_sc, experts)
    y_rows = run_ffn_rows(cfg, offsets, row_src, x, experts)
    assert np.array_equal(y_mat, y_rows)


# ---------------------------------------------------------------- combine

@pytest.mark.parametrize("wt,T,d,I", [("f32", 32, 256, 128), ("bf16", 100, 256, 128), ("bf16", 257, 256, 128),
                                      ("bf16", 1000, 256, 128), ("e4m3", 100, 256, 128), ("e4m3", 257, 256, 128),
                                      # small T, wide d / I: the shared expert splits K (equal and
                                      # unequal split lengths, one and two row tiles, a single token)
                                      ("bf16", 100, 2048, 512), ("bf16", 1, 2048, 512), ("bf16", 130, 1024, 832),
                                      # the large-tile kernels' fused combine epilogues (bf16, e4m3),
                                      # with a ragged last row tile
                                      ("bf16", 600, 512, 256), ("e4m3", 600, 512, 256)])
def test_combine(wt, T, d, I):
    act = "f32" if wt == "f32" else "bf16"
    cfg = synth.Config("comb", seed=31, T=T, d=d, I=I, act=act, wt=wt)
    say(f"[combine] {wt} T={T} d={d} I={I}")
    shared = synth.make_ffn(cfg, 1, (synth.TID_SGATE, synth.TID_SUP, synth.TID_SDOWN))
    x = synth.normal(cfg.seed, synth.TID_X, (T, cfg.d), 1.0, act)
    idx = ids_case("random", T)
    _, _, _, row_of = oracle.dispatch(idx, 256)
    y_perm = synth.normal(cfg.seed, synth.TID_AUX, (cfg.A, cfg.d), 0.1, "f32" if wt == "f32" else "bf16")
    if wt == "e4m3":
        x[5] = 0  # an all-zero row: the shared expert's input tile scale is 1
    g = synth.uniform(cfg.seed, synth.TID_AUX + 1, cfg.A, 0.01, 1.0).reshape(T, 8)
    g = (g / g.sum(axis=1, keepdims=True)).astype(np.float32)
    ds = _lib.desc(T, cfg.d, 256, 8, cfg.I, act, wt)
    sw = {n: (dev(a) if a is not None else None) for n, a in shared.items()}
    fw = _lib.ffn_weights(sw["gate"], sw["up"], sw["down"], sw["s_gate"], sw["s_up"], sw["s_down"])
    y = empty((T, cfg.d), torch.float32)
    ws = empty(_lib.workspace_bytes(ds, _lib.MOE_WS_COMBINE), torch.uint8)
    moe.moe_combine(ds, dev(x), fw, dev(y_perm), dev(row_of), dev(g), y, ws)
    torch.cuda.synchronize()
    yo = oracle.combine(oracle.shape_of(cfg), shared, x, y_perm, row_of, g)
    err = max_rel(host(y), yo)
    say(f"[combine] {wt} T={T}: max rel err {err:.3e}")
    assert err <= TOL[wt], err


# ------------------------------------------------------------ bias update

@pytest.mark.parametrize("T", [32, 2048, 16384])
def test_bias_update_bit_exact(T):
    say(f"[bias] T={T}")
    idx = synth.random_ids(T, synth.TID_IDS, T, 256, 8)
    counts = np.bincount(idx.ravel(), minlength=256).astype(np.int32)
    counts[:4] = T * 8 // 256  # exactly on target: unchanged
    b = synth.uniform(T, synth.TID_AUX, 256, -0.05, 0.05)
    ds = _lib.desc(T, 256, 256, 8, 128, "bf16", "bf16")
    bd = dev(b)
    moe.moe_bias_update(ds, dev(counts), 1e-3, bd)
    torch.cuda.synchronize()
    expect = oracle.bias_update(b, counts, 8, T, 1e-3)
    got = host(bd)
    assert np.array_equal(got, expect)
    assert np.array_equal(got[:4], b[:4])
