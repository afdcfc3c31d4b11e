"""Pins for the oracle's backward with e4m3 expert weights, on the CPU.

Reading under test: every backward GEMM takes e4m3 operands quantised per
1x128 tile along that GEMM's reduction (crackai.dev DeepSeek-V3 summary,
"How It Works": FP8 forward and backward with per-tile scales and FP32
accumulation).  The data-gradient GEMMs reduce along a row (the output
gradient per 1x128 tile of d, the SwiGLU input gradients per tile of I);
the weight-gradient GEMMs reduce over an expert's rows, so each column of a
group of 128 rows (dispatch order) is one tile, quantised from the unrounded
values (and from the bf16 x).

The independent side: torch.autograd in fp64 derives every gradient through
the router, the combine and SwiGLU; the expert linears are custom autograd
Functions whose backward places the quantisers (torch's float8_e4m3fn cast,
itself pinned against the oracle's encoder elsewhere) where the reading puts
them.  An expert with 160 rows and the shared expert over 160 tokens cover
a full and a short 128-row group."""
import numpy as np
import torch

import oracle
import synth
from tests import e4m3_ref

E, K, T, D, I = 16, 4, 160, 256, 128


def q_last(v):
    """1x128 tiles along the last dim, as the forward quantises (power-of-two
    scale at or above amax / 448), dequantised to fp64."""
    q, s = e4m3_ref.quant_last(v.detach())
    t = q.to(torch.float64).reshape(*v.shape[:-1], -1, 128) * s.to(torch.float64)[..., None]
    return t.reshape(v.shape)


def q_cols(v):
    """Each column of each group of 128 consecutive rows as one tile (the
    last group padded with zero rows)."""
    R = v.shape[0]
    pad = (-R) % 128
    vp = torch.cat([v.detach(), torch.zeros((pad, v.shape[1]), dtype=v.dtype)])
    return q_last(vp.T).T[:R]


class QLinear(torch.autograd.Function):
    """out = a_fwd w^T; backward: da = Q_row(g) w, dw = Q_col(g)^T Q_col(a_wg)."""

    @staticmethod
    def forward(ctx, a_fwd, w, a_wg):
        ctx.save_for_backward(w, a_wg)
        return a_fwd @ w.T

    @staticmethod
    def backward(ctx, g):
        w, a_wg = ctx.saved_tensors
        return q_last(g) @ w, q_cols(g).T @ q_cols(a_wg), None


def ste(v, q):
    """Value q(v), derivative the identity (a rounding point of the forward)."""
    return v + (q - v).detach()


def bf16_round(v):
    return v.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def dequant_blocks(codes, scales):
    c = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(e4m3_ref.from_e8m0(scales))
    return c * s.repeat_interleave(128, -2).repeat_interleave(128, -1)


def setup(seed=7):
    cfg = synth.Config("bwd8", seed=seed, T=T, d=D, I=I, wt="e4m3", E=E, k=K)
    x = synth.normal(seed, synth.TID_X, (T, D), 1.0, "bf16")
    wr = synth.normal(seed, synth.TID_WR, (E, D), 0.3, "f32")
    ex = synth.make_ffn(cfg, E, (synth.TID_GATE, synth.TID_UP, synth.TID_DOWN))
    shd = synth.make_ffn(cfg, 1, (synth.TID_SGATE, synth.TID_SUP, synth.TID_SDOWN))
    # experts 0 and 1 for every token (160 rows: a full and a short group), 2 others
    rest = synth.random_ids(seed, synth.TID_IDS, T, E - 2, K - 2) + 2
    idx = np.ascontiguousarray(np.concatenate([np.tile([0, 1], (T, 1)), rest], 1).astype(np.int32))
    dy = synth.normal(seed, synth.TID_AUX, (T, D), 1.0, "f32")
    return cfg, x, wr, ex, shd, idx, dy


def autograd_fp8(x, wr, ex, shd, idx, dy):
    X = torch.tensor(synth.bf16_to_f32(x).astype(np.float64), requires_grad=True)
    WR = torch.tensor(wr.astype(np.float64), requires_grad=True)
    W = {n: dequant_blocks(ex[n], ex["s_" + n]).requires_grad_() for n in ("gate", "up", "down")}
    S = {n: dequant_blocks(shd[n], shd["s_" + n])[0].requires_grad_() for n in ("gate", "up", "down")}
    xq = ste(X, q_last(X))  # the forward's GEMM input: x per 1x128 tile of d

    def ffn(a_fwd, a_raw, wg, wu, wd):
        hraw = torch.nn.functional.silu(QLinear.apply(a_fwd, wg, a_raw)) * QLinear.apply(a_fwd, wu, a_raw)
        return QLinear.apply(ste(hraw, q_last(hraw)), wd, hraw)

    y = ffn(xq, X, S["gate"], S["up"], S["down"])
    s = torch.sigmoid(X @ WR.T)
    ix = torch.tensor(idx, dtype=torch.int64)
    sel = s.gather(1, ix)
    g = sel / sel.sum(1, keepdim=True)
    g.retain_grad()
    flat = ix.reshape(-1)
    yperm = torch.zeros((T * K, D), dtype=torch.float64)
    for e in range(E):
        rows = torch.nonzero(flat == e).reshape(-1)  # dispatch order: ascending t*k + j
        if len(rows) == 0:
            continue
        tok = rows // K
        ye = ffn(xq[tok], X[tok], W["gate"][e], W["up"][e], W["down"][e])
        yperm = yperm.index_put((rows,), ste(ye, bf16_round(ye)))
    y = y + (g.unsqueeze(-1) * yperm.reshape(T, K, D)).sum(1)
    (y * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    return dict(dx=X.grad, dwr=WR.grad, dwg=W["gate"].grad, dwu=W["up"].grad, dwd=W["down"].grad,
                dsg=S["gate"].grad, dsu=S["up"].grad, dsd=S["down"].grad, dg=g.grad)


def rel(a, b):
    b = np.asarray(b, np.float64)
    return np.abs(np.asarray(a, np.float64) - b).max() / max(np.abs(b).max(), 1e-30)


def test_fp8_backward_matches_autograd_with_quantisers():
    cfg, x, wr, ex, shd, idx, dy = setup()
    sh = oracle.shape(T, D, E, K, I, "bf16", "e4m3")
    o = oracle.backward(sh, x, wr, idx, ex, shd, dy)
    a = autograd_fp8(x, wr, ex, shd, idx, dy)
    for n in ("dx", "dwr", "dwg", "dwu", "dwd", "dsg", "dsu", "dsd", "dg"):
        err = rel(o[n], a[n].detach().numpy())
        assert err < 2e-6, (n, err)


def test_fp8_backward_is_near_the_unquantised_one():
    """The quantisers move every gradient by fp8 rounding only: against the
    bf16-weight backward on the same (dequantised) weights, within 10%."""
    cfg, x, wr, ex, shd, idx, dy = setup()
    o8 = oracle.backward(oracle.shape(T, D, E, K, I, "bf16", "e4m3"), x, wr, idx, ex, shd, dy)
    a = autograd_fp8(x, wr, ex, shd, idx, dy)
    # the same forward with no quantiser anywhere
    W = {n: dequant_blocks(ex[n], ex["s_" + n]) for n in ("gate", "up", "down")}
    S = {n: dequant_blocks(shd[n], shd["s_" + n])[0] for n in ("gate", "up", "down")}
    X = torch.tensor(synth.bf16_to_f32(x).astype(np.float64), requires_grad=True)
    WR = torch.tensor(wr.astype(np.float64))
    f = lambda v, e: (torch.nn.functional.silu(v @ W["gate"][e].T) * (v @ W["up"][e].T)) @ W["down"][e].T
    y = (torch.nn.functional.silu(X @ S["gate"].T) * (X @ S["up"].T)) @ S["down"].T
    s = torch.sigmoid(X @ WR.T)
    ix = torch.tensor(idx, dtype=torch.int64)
    sel = s.gather(1, ix)
    g = sel / sel.sum(1, keepdim=True)
    y = y + torch.stack([sum(g[t, j] * f(X[t:t + 1], int(ix[t, j]))[0] for j in range(K)) for t in range(T)])
    (y * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    assert rel(o8["dx"], X.grad.numpy()) < 0.1
    assert 1e-4 < rel(o8["dx"], X.grad.numpy())  # the quantisers do act
    del a


def test_fp8_shared_column_mode_equals_the_full_gradients():
    """The reduced mode the full-size check uses, with e4m3 weights: the
    shared expert's weight gradients for a few SwiGLU columns over all 160
    tokens (a full and a short 128-token group) equal the full run's bit for
    bit; every operand tile is one column of a group, so cutting the columns
    changes no tile."""
    cfg, x, wr, ex, shd, idx, dy = setup()
    sh = oracle.shape(T, D, E, K, I, "bf16", "e4m3")
    full = oracle.backward(sh, x, wr, idx, ex, shd, dy)
    cols = [0, 77, I - 1]
    part = oracle.backward_shared_cols(sh, x, shd, dy, cols)
    assert np.array_equal(part["dsg"], full["dsg"][cols])
    assert np.array_equal(part["dsu"], full["dsu"][cols])
    assert np.array_equal(part["dsd"], full["dsd"][:, cols])
