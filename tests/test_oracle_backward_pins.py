"""Pins for the oracle's backward (gradients of the layer output), on the CPU.

The oracle's hand-derived gradients are checked against torch.autograd in
fp64 on the same forward written with plain torch ops (an independent
derivation by a library): tightly with fp32 weights (where the oracle's only
roundings are to fp32), and to the bf16 rounding level with bf16 weights
(where the oracle rounds the backward GEMM inputs like the forward rounds h).
Also: the choice carries no gradient (gradients for a fixed routing equal the
autograd ones even though the choice depends on x), the bias appears nowhere
in the gradients, and the combine-weight gradient dg is dy . y_perm."""
import numpy as np
import pytest
import torch

import oracle
import synth

E, K = 16, 4


def setup(act, wt, T=6, d=32, I=16, seed=3):
    cfg = synth.Config("bwd", seed=seed, T=T, d=d, I=I, act=act, wt=wt, E=E, k=K)
    x = synth.normal(seed, synth.TID_X, (T, d), 1.0, act)
    wr = synth.normal(seed, synth.TID_WR, (E, d), 0.3, "f32")
    experts = synth.make_ffn(cfg, E, (synth.TID_GATE, synth.TID_UP, synth.TID_DOWN))
    shared = synth.make_ffn(cfg, 1, (synth.TID_SGATE, synth.TID_SUP, synth.TID_SDOWN))
    bias = synth.uniform(seed, synth.TID_BIAS, E, -0.05, 0.05)
    sh = oracle.shape(T, d, E, K, I, act, wt)
    idx, _, _, _ = oracle.route(sh, x, wr, bias)
    dy = synth.normal(seed, synth.TID_AUX, (T, d), 1.0, "f32")
    return cfg, sh, x, wr, experts, shared, bias, idx, dy


def dec(a, dt):
    if dt == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def autograd(x, wr, experts, shared, idx, dy, dt_x, dt_w):
    """fp64 autograd of y = shared(x) + sum_j g_j FFN_{e_j}(x), g = s_sel / sum s_sel."""
    t = lambda a, dt: torch.tensor(dec(a, dt), dtype=torch.float64, requires_grad=True)
    X, WR = t(x, dt_x), torch.tensor(wr.astype(np.float64), requires_grad=True)
    G, U, D = t(experts["gate"], dt_w), t(experts["up"], dt_w), t(experts["down"], dt_w)
    SG, SU, SD = t(shared["gate"], dt_w), t(shared["up"], dt_w), t(shared["down"], dt_w)
    ffn = lambda a, g_, u_, d_: (torch.nn.functional.silu(a @ g_.T) * (a @ u_.T)) @ d_.T
    s = torch.sigmoid(X @ WR.T)
    ix = torch.tensor(idx, dtype=torch.int64)
    sel = s.gather(1, ix)
    g = sel / sel.sum(1, keepdim=True)
    y = ffn(X, SG[0], SU[0], SD[0])
    routed = []
    for tk in range(X.shape[0]):
        r = 0
        for j in range(ix.shape[1]):
            e = int(ix[tk, j])
            r = r + g[tk, j] * ffn(X[tk:tk + 1], G[e], U[e], D[e])[0]
        routed.append(r)
    y = y + torch.stack(routed)
    (y * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    return dict(dx=X.grad, dwr=WR.grad, dwg=G.grad, dwu=U.grad, dwd=D.grad, dsg=SG.grad[0], dsu=SU.grad[0],
                dsd=SD.grad[0])


def rel(a, b):
    b = np.asarray(b, np.float64)
    return np.abs(np.asarray(a, np.float64) - b).max() / max(np.abs(b).max(), 1e-30)


def test_backward_matches_autograd_fp32():
    cfg, sh, x, wr, ex, shd, bias, idx, dy = setup("f32", "f32")
    o = oracle.backward(sh, x, wr, idx, ex, shd, dy)
    a = autograd(x, wr, ex, shd, idx, dy, "f32", "f32")
    for n in ("dx", "dwr", "dwg", "dwu", "dwd", "dsg", "dsu", "dsd"):
        assert rel(o[n], a[n].numpy()) < 2e-6, n


def test_backward_matches_autograd_bf16_to_rounding_level():
    cfg, sh, x, wr, ex, shd, bias, idx, dy = setup("bf16", "bf16")
    o = oracle.backward(sh, x, wr, idx, ex, shd, dy)
    a = autograd(x, wr, ex, shd, idx, dy, "bf16", "bf16")
    for n in ("dx", "dwr", "dwg", "dwu", "dwd", "dsg", "dsu", "dsd"):
        assert rel(o[n], a[n].numpy()) < 3e-2, n


def test_dg_is_dy_dot_routed_output():
    cfg, sh, x, wr, ex, shd, bias, idx, dy = setup("f32", "f32")
    o = oracle.backward(sh, x, wr, idx, ex, shd, dy)
    _, offsets, row_src, row_of = oracle.dispatch(idx, E)
    y_perm = oracle.expert_ffn(sh, ex, offsets, np.ascontiguousarray(x[row_src // K]))
    want = np.einsum("tjn,tn->tj", y_perm[row_of].reshape(cfg.T, K, cfg.d).astype(np.float64), dy)
    assert rel(o["dg"], want) < 1e-6


def test_bias_enters_only_through_the_choice():
    """A bias change that leaves the routing as it is leaves every gradient
    as it is (the bias gets no gradient of its own)."""
    cfg, sh, x, wr, ex, shd, bias, idx, dy = setup("f32", "f32")
    b2 = (bias + np.float32(1e-6)).astype(np.float32)
    idx2, _, _, _ = oracle.route(sh, x, wr, b2)
    assert np.array_equal(idx, idx2), "the 1e-6 shift changed the routing for this seed"
    o1 = oracle.backward(sh, x, wr, idx, ex, shd, dy)
    o2 = oracle.backward(sh, x, wr, idx2, ex, shd, dy)
    for n in o1:
        assert np.array_equal(o1[n], o2[n]), n


def test_sampled_modes_equal_the_full_gradients():
    """The reduced modes full-size checks use: dx and dg of a token subset
    equal the full run's rows (they are per-token), and an expert's weight
    gradients from only the tokens that chose it equal the full run's slice
    (no other token's row enters them)."""
    cfg, sh, x, wr, ex, shd, bias, idx, dy = setup("bf16", "bf16", T=24)
    full = oracle.backward(sh, x, wr, idx, ex, shd, dy)
    toks = np.array([1, 5, 17, 23])
    sub = oracle.shape(len(toks), cfg.d, E, K, cfg.I, "bf16", "bf16")
    part = oracle.backward(sub, np.ascontiguousarray(x[toks]), wr, np.ascontiguousarray(idx[toks]), ex, shd,
                           np.ascontiguousarray(dy[toks]), weight_grads=False)
    assert set(part) == {"dx", "dg"}
    assert np.array_equal(part["dx"], full["dx"][toks]) and np.array_equal(part["dg"], full["dg"][toks])
    e = int(np.bincount(idx.ravel(), minlength=E).argmax())
    mine = np.flatnonzero((idx == e).any(1))
    assert 0 < len(mine) < cfg.T
    sub = oracle.shape(len(mine), cfg.d, E, K, cfg.I, "bf16", "bf16")
    one = oracle.backward(sub, np.ascontiguousarray(x[mine]), wr, np.ascontiguousarray(idx[mine]), ex, shd,
                          np.ascontiguousarray(dy[mine]), weight_grads=e)
    for n in ("dwr", "dwg", "dwu", "dwd"):
        assert np.allclose(one[n][0], full[n][e], rtol=1e-6, atol=1e-7 * np.abs(full[n][e]).max()), n
    assert np.array_equal(one["dx"], full["dx"][mine])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_shared_column_mode_equals_the_full_gradients(dt):
    """The reduced mode the full-size check of the shared expert uses: its
    weight gradients for a few SwiGLU columns (rows of dsg and dsu, columns
    of dsd) over all tokens equal the full run's bit for bit."""
    cfg, sh, x, wr, ex, shd, bias, idx, dy = setup(dt, dt, T=24)
    full = oracle.backward(sh, x, wr, idx, ex, shd, dy)
    cols = [0, 5, cfg.I - 1]
    part = oracle.backward_shared_cols(sh, x, shd, dy, cols)
    assert np.array_equal(part["dsg"], full["dsg"][cols])
    assert np.array_equal(part["dsu"], full["dsu"][cols])
    assert np.array_equal(part["dsd"], full["dsd"][:, cols])
