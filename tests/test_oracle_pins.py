"""Pins for the CPU oracle: checks against what the pages and the mathematics fix,
never against the oracle's own formulas retyped.

Kinds of pin used here:
  * library routines (torch's bf16 / float8_e4m3fn casts, scipy's expit,
    numpy's stable argsort and cumsum) on the same inputs;
  * closed forms (zero router -> affinity exactly 0.5; one-hot token -> logits
    are a column of the router; identity experts -> y = silu(c x) x);
  * the pages' worked example and the hand-derived bias step (tests/golden);
  * brute force on tiny inputs: a full sort for the selection and a dense
    all-expert FFN, masked by the routing, written with torch library ops;
  * invariants (weights sum to 1, loads sum to T*k, no token dropped);
  * a negative control: the softmax-over-biased-logits scoring printed on
    one of the pages must NOT match the oracle.
"""
import json
import os

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle
import synth
from tests import e4m3_ref

torch.set_num_threads(4)


# ----------------------------------------------------------------- helpers

def bf16_round_t(v: torch.Tensor) -> torch.Tensor:
    """Library bf16 rounding (torch, RNE) of fp64 values via fp32."""
    return v.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def e4m3_tiles_t(v: torch.Tensor) -> torch.Tensor:
    """Library e4m3 quantisation per 1x128 tile (torch cast), dequantised to fp64."""
    shp = v.shape
    q, s = e4m3_ref.quant_last(v.reshape(-1, 128))
    return (q.to(torch.float64) * s.to(torch.float64)).reshape(shp)


def dequant_weights(w, s, dt):
    """[G, N, K] weights (f32 / bf16 bits / e4m3 codes + [G,N/128,K/128] scales) -> fp64 torch."""
    if dt == "f32":
        return torch.from_numpy(w.astype(np.float64))
    if dt == "bf16":
        return torch.from_numpy(synth.bf16_to_f32(w).astype(np.float64))
    q = torch.from_numpy(w).view(torch.float8_e4m3fn).to(torch.float64)
    sc = torch.from_numpy(e4m3_ref.from_e8m0(s))
    sc = sc.repeat_interleave(128, dim=1).repeat_interleave(128, dim=2)
    return q * sc


def x_values(x, act):
    return synth.bf16_to_f32(x).astype(np.float64) if act == "bf16" else x.astype(np.float64)


def brute_forward(cfg, inp, bias=None):
    """Dense brute force of the whole layer on all tokens (tiny shapes only):
    full-sort selection and every expert applied to every token, masked."""
    E, k, T = cfg.E, cfg.k, cfg.T
    b = inp["bias"] if bias is None else bias
    xr = torch.from_numpy(x_values(inp["x"], cfg.act))
    wr = torch.from_numpy(inp["wr"].astype(np.float64))
    s = torch.from_numpy(expit((xr @ wr.T).numpy()))
    v32 = s.to(torch.float32).numpy() + b  # fp32 decision
    idx = np.zeros((T, k), np.int64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -v32[t]))  # by score desc, then id asc
        idx[t] = np.sort(order[:k])
    sel = torch.gather(s, 1, torch.from_numpy(idx))
    g = sel / sel.sum(dim=1, keepdim=True)
    mask = torch.zeros(T, E, dtype=torch.float64)
    mask.scatter_(1, torch.from_numpy(idx), g)
    a = xr if cfg.wt != "e4m3" else e4m3_tiles_t(xr)

    def rnd_h(h):
        if cfg.wt == "f32":
            return h.to(torch.float32).to(torch.float64)
        if cfg.wt == "bf16":
            return bf16_round_t(h)
        return e4m3_tiles_t(h)

    def rnd_y(y):
        return y.to(torch.float32).to(torch.float64) if cfg.wt == "f32" else bf16_round_t(y)

    def ffn(w, G):
        Wg = dequant_weights(w["gate"], w["s_gate"], cfg.wt)
        Wu = dequant_weights(w["up"], w["s_up"], cfg.wt)
        Wd = dequant_weights(w["down"], w["s_down"], cfg.wt)
        outs = []
        for e in range(G):
            h = rnd_h(torch.nn.functional.silu(a @ Wg[e].T) * (a @ Wu[e].T))
            outs.append(h @ Wd[e].T)
        return torch.stack(outs)  # [G, T, d]

    routed = rnd_y(ffn(inp["experts"], E))
    shared = ffn(inp["shared"], 1)[0]
    y = shared + torch.einsum("te,etd->td", mask, routed)
    return idx, g.numpy(), y.numpy()


def tiny_cfg(act="bf16", wt="bf16", T=5, d=256, I=128, E=16, k=4, seed=11, bias="uniform"):
    return synth.Config("tiny", seed=seed, T=T, d=d, I=I, E=E, k=k, act=act, wt=wt, bias=bias)


def sh_of(cfg):
    return oracle.shape_of(cfg)


# ------------------------------------------------------------------ codecs

def test_bf16_encode_matches_torch_including_ties():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    # force exact ties (lower half = 0x8000) on both parities of the upper half
    bits[:4000] = (bits[:4000] & 0xFFFF0000) | 0x8000
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3e38)]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = np.array([oracle.bf16_encode(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(mine, ref)


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.e4m3_decode(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2  # 0x7F, 0xFF
    assert np.array_equal(mine[~nan], ref[~nan])
    assert oracle.e4m3_decode(0x7E) == 448.0 and oracle.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_encode_matches_torch_rne_and_saturates():
    vals = np.array([oracle.e4m3_decode(c) for c in range(0x7F)])
    mids = (vals[:-1] + vals[1:]) / 2  # exact ties between neighbouring codes
    rng = np.random.default_rng(1)
    rand = rng.uniform(-448, 448, 20000) * rng.choice([1, 1e-1, 1e-2, 1e-3], 20000)
    test = np.concatenate([vals, mids, -mids, rand]).astype(np.float32)
    ref = torch.from_numpy(test).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([oracle.e4m3_encode(float(v)) for v in test], dtype=np.uint8)
    assert np.array_equal(mine, ref)
    for v in (448.5, 470.0, 1e6):
        assert oracle.e4m3_encode(v) == 0x7E and oracle.e4m3_encode(-v) == 0xFE


def test_tile_quantisation_matches_torch_cast():
    x = synth.normal(5, synth.TID_AUX, (7, 384), 1.0, "bf16")
    q, s = oracle.quant_e4m3_rows(x, "bf16")
    xv = torch.from_numpy(synth.bf16_to_f32(x)).reshape(7, 3, 128)
    amax = xv.abs().amax(dim=2)
    ref_q, ref_s = e4m3_ref.quant_last(xv.reshape(7, 384))
    assert s.dtype == np.uint8 and np.array_equal(s, e4m3_ref.to_e8m0(ref_s))
    assert np.array_equal(q, ref_q.view(torch.uint8).reshape(7, 384).numpy())
    # the scale is a power of two with amax / scale in (224, 448]: the tile's
    # largest value lands in the top binade of e4m3
    r = amax.numpy() / e4m3_ref.from_e8m0(s)
    assert (r > 224).all() and (r <= 448).all()
    # an all-zero tile gets scale 1 (E8M0 byte 127) and zero codes
    z = np.zeros((1, 128), np.float32)
    qz, sz = oracle.quant_e4m3_rows(z, "f32")
    assert sz[0, 0] == 127 and not qz.any()


def test_e8m0_codec_matches_ldexp():
    """The oracle's E8M0 decoder over all 256 bytes: 2^(e - 127) by numpy's
    ldexp for e = 0 .. 254, NaN for 255 (OCP MX scale format)."""
    for e in range(255):
        assert oracle.e8m0_decode(e) == float(np.ldexp(1.0, e - 127)), e
    assert np.isnan(oracle.e8m0_decode(255))


# ------------------------------------------------------------------ router

def test_zero_router_gives_half_and_lowest_ids():
    """W_r = 0: every affinity is exactly sigmoid(0) = 1/2; with b = 0 all
    biased scores tie and the lower ids win; weights are 1/k each."""
    T, d, E, k = 3, 64, 256, 8
    x = synth.normal(1, synth.TID_AUX, (T, d), 1.0, "f32")
    wr = np.zeros((E, d), np.float32)
    sh = oracle.shape(T, d, E, k, 64, "f32", "f32")
    idx, g, gap, s = oracle.route(sh, x, wr, np.zeros(E, np.float32), want_s=True)
    assert np.all(s == 0.5)
    assert np.array_equal(idx, np.tile(np.arange(8), (T, 1)))
    assert np.all(g == np.float32(1 / 8)) and np.all(gap == 0.0)


def test_one_hot_token_logits_are_router_column():
    """x = e_j: logit of expert i is W_r[i, j] exactly, so s = expit(W_r[:, j])."""
    d, E, k = 32, 256, 8
    wr = synth.normal(2, synth.TID_AUX, (E, d), 0.5, "f32")
    x = np.zeros((d, d), np.float32)
    np.fill_diagonal(x, 1.0)
    sh = oracle.shape(d, d, E, k, 64, "f32", "f32")
    _, _, _, s = oracle.route(sh, x, wr, np.zeros(E, np.float32), want_s=True)
    np.testing.assert_allclose(s, expit(wr.T.astype(np.float64)), rtol=1e-15, atol=0)


def test_zero_bias_is_plain_topk():
    """With b = 0 the choice is the plain top-k of the affinities (torch.topk)."""
    cfg = synth.CONFIGS[2].with_(T=64, d=512, bias="zero")
    x, wr, bias = synth.make_router(cfg)
    idx, _, gap, s = oracle.route(oracle.shape_of(cfg), x, wr, bias, want_s=True)
    ref = torch.topk(torch.from_numpy(s.astype(np.float32)), 8, dim=1).indices.numpy()
    ok = gap > 1e-6  # torch's order between exactly equal fp32 scores is unspecified
    assert ok.sum() >= 60
    assert np.array_equal(idx[ok], np.sort(ref, axis=1)[ok])


def test_worked_example_rank9_joins_with_bias(golden_dir):
    """DeepSeek V3 From Scratch, 'Worked example': rank-9 expert + 0.05 joins."""
    G = json.load(open(os.path.join(golden_dir, "worked_example_rank9.json")))
    E, k = G["E"], G["k"]
    for case in G["cases"]:
        aff = np.full(E, G["others_affinity"])
        aff[G["top8_experts_by_affinity"]] = G["top8_affinities"]
        aff[G["rank9_expert"]] = case["rank9_affinity"]
        logit = np.log(aff / (1 - aff))  # inverse sigmoid
        x = np.ones((1, 1), np.float32)
        wr = logit.astype(np.float32)[:, None]
        sh = oracle.shape(1, 1, E, k, 64, "f32", "f32")
        b0 = np.zeros(E, np.float32)
        idx0, g0, _, s = oracle.route(sh, x, wr, b0, want_s=True)
        assert list(idx0[0]) == sorted(G["top8_experts_by_affinity"])
        b = b0.copy()
        b[G["rank9_expert"]] = case["bias_on_rank9"]
        idx1, g1, _, _ = oracle.route(sh, x, wr, b)
        chosen = set(idx1[0])
        if case["joins"]:
            expect = (set(G["top8_experts_by_affinity"]) - {G["rank8_expert"]}) | {G["rank9_expert"]}
        else:
            expect = set(G["top8_experts_by_affinity"])
        assert chosen == expect
        # weights come from the unbiased affinities of the chosen set
        sv = s[0, idx1[0]]
        np.testing.assert_allclose(g1[0], sv / sv.sum(), rtol=1e-7)
        assert abs(float(g1[0].astype(np.float64).sum()) - 1) < 1e-6


def test_weights_do_not_depend_on_bias_given_the_set():
    """Bias shifts the choice only: two biases that pick the same experts give
    identical weights (kbwen.com feed, 'A bias term for each expert')."""
    cfg = synth.CONFIGS[2].with_(T=32, d=256)
    x, wr, bias = synth.make_router(cfg)
    sh = oracle.shape_of(cfg)
    idx1, g1, _, _ = oracle.route(sh, x, wr, bias)
    idx2, g2, _, _ = oracle.route(sh, x, wr, bias + np.float32(1.0))  # uniform shift keeps the order
    same = np.all(idx1 == idx2, axis=1)
    assert same.mean() > 0.9
    assert np.array_equal(g1[same], g2[same])


def test_route_brute_force_tiny():
    for seed in range(4):
        for E, k in ((16, 4), (16, 1), (9, 8), (8, 8)):
            cfg = tiny_cfg(act="f32", wt="f32", T=4, d=8, E=E, k=k, seed=seed)
            x, wr, bias = synth.make_router(cfg.with_(std_w=0.5))
            idx, g, gap, s = oracle.route(oracle.shape_of(cfg), x, wr, bias, want_s=True)
            s_ref = expit(x.astype(np.float64) @ wr.astype(np.float64).T)
            np.testing.assert_allclose(s, s_ref, rtol=1e-14)
            v32 = s_ref.astype(np.float32) + bias
            v64 = s_ref + bias.astype(np.float64)
            for t in range(cfg.T):
                order = np.argsort(-v32[t], kind="stable")  # equal scores keep id order
                assert list(idx[t]) == sorted(order[:k])
                sel = s_ref[t, idx[t]]
                np.testing.assert_allclose(g[t], sel / sel.sum(), rtol=1e-7)
                vs = np.sort(v64[t])[::-1]
                assert gap[t] == (vs[k - 1] - vs[k] if k < E else np.inf)


def test_negative_control_softmax_of_biased_logits_differs():
    """One page scores with a softmax over the biased top-k linear logits.
    The oracle must not: its weights are renormalised sigmoid affinities."""
    cfg = synth.CONFIGS[2].with_(T=16, d=256)
    x, wr, bias = synth.make_router(cfg)
    idx, g, _, _ = oracle.route(oracle.shape_of(cfg), x, wr, bias)
    logits = torch.from_numpy(synth.bf16_to_f32(x).astype(np.float64)) @ torch.from_numpy(wr.astype(np.float64)).T
    biased = logits + torch.from_numpy(bias.astype(np.float64))
    top = torch.topk(biased, 8, dim=1)
    sm = torch.softmax(top.values, dim=1)
    idx_p = np.sort(top.indices.numpy(), axis=1)
    g_p = np.take_along_axis(sm.numpy(), np.argsort(top.indices.numpy(), axis=1), axis=1)
    assert np.abs(g_p - g).max() > 1e-2
    assert not np.array_equal(idx_p, idx) or np.abs(g_p - g).max() > 1e-2


# ---------------------------------------------------------------- dispatch

def test_dispatch_matches_stable_argsort_and_invariants():
    T, E, k = 300, 256, 8
    idx = synth.random_ids(3, synth.TID_IDS, T, E, k)
    assert all(len(set(r)) == k for r in idx)  # k distinct experts per token
    counts, offsets, row_src, row_of = oracle.dispatch(idx, E)
    assert counts.sum() == T * k  # no token dropped
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(row_src, np.argsort(idx.ravel(), kind="stable"))
    assert np.array_equal(row_of[row_src], np.arange(T * k))


def test_dispatch_degenerate_all_tokens_same_experts():
    T, E, k = 50, 256, 8
    idx = np.tile(np.arange(8, dtype=np.int32), (T, 1))
    counts, offsets, row_src, _ = oracle.dispatch(idx, E)
    assert np.all(counts[:8] == T) and not counts[8:].any()
    assert np.array_equal(row_src[:T], np.arange(T) * k)  # expert 0: tokens in order


# -------------------------------------------------------------- bias update

def test_bias_update_by_hand(golden_dir):
    G = json.load(open(os.path.join(golden_dir, "update_bias_by_hand.json")))
    b_in = np.array(G["bias_in"], np.float32)
    out = oracle.bias_update(b_in, np.array(G["counts"]), G["k"], G["T"], G["gamma"])
    sign = np.array(G["expected_sign"], np.float32)
    expect = b_in + np.float32(G["gamma"]) * sign  # numpy fp32 arithmetic
    assert out.dtype == np.float32 and np.array_equal(out, expect)
    assert out[0] == b_in[0] and out[3] == b_in[3]  # on target: unchanged


def test_bias_update_matches_pages_torch_expression():
    """The page's expression bias + step * sign(target - load), load = c/T,
    target = k/E, evaluated with torch in fp64 (exact for power-of-two T)."""
    T, E, k = 1024, 256, 8
    idx = synth.random_ids(4, synth.TID_IDS, T, E, k)
    counts = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    b = synth.uniform(4, synth.TID_AUX, E, -0.05, 0.05)
    out = oracle.bias_update(b, counts, k, T)
    load = torch.from_numpy(counts.astype(np.float64)) / T
    sgn = torch.sign(torch.tensor(k / E, dtype=torch.float64) - load).to(torch.float32)
    ref = torch.from_numpy(b) + torch.tensor(1e-3, dtype=torch.float32) * sgn
    assert np.array_equal(out, ref.numpy())
    assert (out != b).sum() == (counts != k * T // E).sum()


def test_bias_stays_within_n_gamma():
    cfg = synth.CONFIGS[4].with_(T=256, d=128, steps=10)
    x, wr, bias = synth.make_router(cfg)
    sh = oracle.shape_of(cfg)
    b = bias.copy()
    for n in range(1, cfg.steps + 1):
        idx, _, _, _ = oracle.route(sh, x, wr, b)
        counts, *_ = oracle.dispatch(idx, cfg.E)
        assert counts.sum() == cfg.T * cfg.k
        b2 = oracle.bias_update(b, counts, cfg.k, cfg.T)
        step = np.abs(b2.astype(np.float64) - b)
        assert np.all((step == 0) | (np.abs(step - 1e-3) < 1e-9))
        b = b2
        assert np.all(np.abs(b) <= n * 1e-3 * (1 + 1e-5))


# ------------------------------------------------------ expert FFN, combine

@pytest.mark.parametrize("act,wt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "e4m3")])
def test_forward_brute_force_dense(act, wt):
    cfg = tiny_cfg(act=act, wt=wt, T=5, d=256, I=128, E=16, k=4)
    inp = synth.make_inputs(cfg)
    sh = sh_of(cfg)
    idx, g, gap, y = oracle.forward(sh, inp["x"], inp["wr"], inp["bias"], inp["experts"], inp["shared"])
    idx_b, g_b, y_b = brute_forward(cfg, inp)
    assert np.array_equal(idx, idx_b)
    np.testing.assert_allclose(g, g_b, rtol=2e-7)
    # fp64 vs fp64 with the same rounding points: only the summation order and
    # the final fp32 rounding differ
    err = np.abs(y - y_b).max() / np.abs(y_b).max()
    assert err < 1e-6, err


@pytest.mark.parametrize("act,wt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "e4m3")])
def test_staged_path_equals_forward(act, wt):
    """route -> dispatch -> expert FFN on permuted rows -> combine gives the
    same y as the per-token forward (the grouping must not change values)."""
    cfg = tiny_cfg(act=act, wt=wt, T=6, d=256, I=128, E=16, k=4, seed=5)
    inp = synth.make_inputs(cfg)
    sh = sh_of(cfg)
    idx, g, _, y = oracle.forward(sh, inp["x"], inp["wr"], inp["bias"], inp["experts"], inp["shared"])
    idx2, g2, _, _ = oracle.route(sh, inp["x"], inp["wr"], inp["bias"])
    assert np.array_equal(idx, idx2) and np.array_equal(g, g2)
    counts, offsets, row_src, row_of = oracle.dispatch(idx2, cfg.E)
    tok = row_src // cfg.k
    if wt == "e4m3":
        q, s = oracle.quant_e4m3_rows(inp["x"], act)
        a_rows, a_sc = np.ascontiguousarray(q[tok]), np.ascontiguousarray(s[tok])
    else:
        a_rows, a_sc = np.ascontiguousarray(inp["x"][tok]), None
    y_perm = oracle.expert_ffn(sh, inp["experts"], offsets, a_rows, a_sc)
    y2 = oracle.combine(sh, inp["shared"], inp["x"], y_perm, row_of, g2)
    np.testing.assert_allclose(y2, y, rtol=0, atol=1e-6 * np.abs(y).max())


def test_zero_input_gives_zero_output():
    cfg = tiny_cfg(T=3)
    inp = synth.make_inputs(cfg)
    x0 = np.zeros_like(inp["x"])
    _, _, _, y = oracle.forward(sh_of(cfg), x0, inp["wr"], inp["bias"], inp["experts"], inp["shared"])
    assert not y.any()  # silu(0) = 0


def test_zero_up_projection_leaves_only_shared():
    cfg = tiny_cfg(T=3, wt="bf16")
    inp = synth.make_inputs(cfg)
    sh = sh_of(cfg)
    ex = dict(inp["experts"], up=np.zeros_like(inp["experts"]["up"]))
    _, _, _, y = oracle.forward(sh, inp["x"], inp["wr"], inp["bias"], ex, inp["shared"])
    no_sh = dict(inp["shared"], down=np.zeros_like(inp["shared"]["down"]))
    _, _, _, y_routed = oracle.forward(sh, inp["x"], inp["wr"], inp["bias"], inp["experts"], no_sh)
    _, _, _, y_full = oracle.forward(sh, inp["x"], inp["wr"], inp["bias"], inp["experts"], inp["shared"])
    np.testing.assert_allclose(y_full - y_routed, y, rtol=0, atol=1e-6 * np.abs(y).max())


def test_identity_experts_closed_form():
    """d = I, W_gate = c*Id, W_up = W_down = Id for every expert (routed and
    shared): h = silu(c x) * x, and because the k weights sum to 1 the routed
    part equals one expert's output whatever the routing.  fp32 storage."""
    d = I = 128
    E, k, T, c = 16, 4, 5, 0.7
    cfg = tiny_cfg(act="f32", wt="f32", T=T, d=d, I=I, E=E, k=k)
    x, wr, bias = synth.make_router(cfg)
    eye = np.eye(d, dtype=np.float32)
    ex = dict(gate=np.stack([c * eye] * E), up=np.stack([eye] * E), down=np.stack([eye] * E),
              s_gate=None, s_up=None, s_down=None)
    shd = dict(gate=(c * eye)[None], up=eye[None], down=eye[None], s_gate=None, s_up=None, s_down=None)
    _, g, _, y = oracle.forward(sh_of(cfg), x, wr, bias, ex, shd)
    xd = x.astype(np.float64)
    z = c * xd
    h = z * expit(z) * xd
    h32 = h.astype(np.float32).astype(np.float64)
    expect = h32 + h32.astype(np.float32).astype(np.float64) * g.astype(np.float64).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(y, expect, rtol=2e-7, atol=1e-7)


def test_down_projection_scales_linearly():
    """Doubling every W_down (exact in bf16) doubles y exactly."""
    cfg = tiny_cfg(T=4)
    inp = synth.make_inputs(cfg)
    sh = sh_of(cfg)

    def dbl(w):
        v = synth.bf16_to_f32(w) * 2
        return (v.view(np.uint32) >> 16).astype(np.uint16)
    ex = dict(inp["experts"], down=dbl(inp["experts"]["down"]))
    shd = dict(inp["shared"], down=dbl(inp["shared"]["down"]))
    _, _, _, y1 = oracle.forward(sh, inp["x"], inp["wr"], inp["bias"], inp["experts"], inp["shared"])
    _, _, _, y2 = oracle.forward(sh, inp["x"], inp["wr"], inp["bias"], ex, shd)
    assert np.array_equal(y2, 2 * y1)


def test_identity_experts_closed_form_bf16():
    """bf16 storage with identity experts (W_gate = c*Id, c = 0.75 exact in
    bf16): h = bf16(silu(c x) x); W_down = Id reproduces h exactly, so
    y = h + bf16(h) * sum_j g_j, which pins the rounding of h to bf16."""
    d = I = 128
    E, k, T, c = 16, 4, 5, 0.75
    cfg = tiny_cfg(act="bf16", wt="bf16", T=T, d=d, I=I, E=E, k=k)
    x, wr, bias = synth.make_router(cfg)
    one = np.uint16(0x3F80)  # 1.0 in bf16
    eye = np.where(np.eye(d, dtype=bool), one, np.uint16(0)).astype(np.uint16)
    ceye = np.where(np.eye(d, dtype=bool), np.uint16(0x3F40), np.uint16(0)).astype(np.uint16)  # 0.75
    ex = dict(gate=np.stack([ceye] * E), up=np.stack([eye] * E), down=np.stack([eye] * E),
              s_gate=None, s_up=None, s_down=None)
    shd = dict(gate=ceye[None], up=eye[None], down=eye[None], s_gate=None, s_up=None, s_down=None)
    _, g, _, y = oracle.forward(sh_of(cfg), x, wr, bias, ex, shd)
    xd = torch.from_numpy(synth.bf16_to_f32(x).astype(np.float64))
    h = bf16_round_t(torch.nn.functional.silu(c * xd) * xd).numpy()
    expect = h + h * g.astype(np.float64).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(y, expect, rtol=1e-7, atol=1e-9)
