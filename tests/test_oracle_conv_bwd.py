"""Pins of the oracle's ShortConv reverse mode (oracle.shortconv_dual_bwd)
against what the forward's definition and calculus fix, independently of its
loops:
  * central finite differences of L = <dy, y> + <dy~, y~> through the
    oracle's forward, for every input (x, x~, weight, bias), with and without
    the SiLU activation;
  * the adjoint identity: without activation and bias the forward is linear in
    (x, x~) and in the weight, so <dy, y> + <dy~, y~> = <dx, x> + <dx~, x~>
    = <dweight, weight> exactly (up to rounding);
  * a one-hot output gradient returns the taps: dx holds the weights at the
    positions the output read, and dweight the values it read;
  * structure: noisy prompt rows receive no gradient, the noisy output
    gradient's prompt rows are ignored, and no gradient crosses documents.
"""
import numpy as np
import pytest

import oracle

CU = [0, 11, 11, 20, 30, 36]
PROMPTS = [4, 0, 0, 8, 4]


def draw(seed, T, C, W, bias=True):
    rng = np.random.default_rng(seed)
    x, xn = rng.standard_normal((T, C)), rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    b = rng.standard_normal(C) if bias else None
    dy, dyn = rng.standard_normal((T, C)), rng.standard_normal((T, C))
    return x, xn, w, b, dy, dyn


def loss(B, x, xn, w, b, dy, dyn, act):
    y, yn = oracle.shortconv_dual(CU, PROMPTS, B, x, xn, w, bias=b, activation=act)
    return float(np.sum(dy * y) + np.sum(dyn * yn))


@pytest.mark.parametrize("W,B,act,bias", [(1, 2, 0, False), (3, 2, 1, True), (4, 4, 0, True), (4, 4, 1, False),
                                          (6, 2, 1, True)])
def test_finite_differences(W, B, act, bias):
    T, C = CU[-1], 3
    x, xn, w, b, dy, dyn = draw(100 + W + B, T, C, W, bias)
    dx, dxn, dw, db = oracle.shortconv_dual_bwd(CU, PROMPTS, B, x, xn, w, dy, dyn, bias=b, activation=act)
    h = 1e-6
    rng = np.random.default_rng(7)
    args = {"x": x, "xn": xn, "w": w, "b": b}
    grads = {"x": dx, "xn": dxn, "w": dw, "b": db}
    for name in ("x", "xn", "w") + (("b",) if bias else ()):
        for _ in range(3):
            d = rng.standard_normal(args[name].shape)
            up = dict(args); up[name] = args[name] + h * d
            dn = dict(args); dn[name] = args[name] - h * d
            fd = (loss(B, up["x"], up["xn"], up["w"], up["b"], dy, dyn, act)
                  - loss(B, dn["x"], dn["xn"], dn["w"], dn["b"], dy, dyn, act)) / (2 * h)
            an = float(np.sum(grads[name] * d))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)
    # every weight entry on its own
    for c in range(C):
        for j in range(W):
            up = w.copy(); up[c, j] += h
            dn = w.copy(); dn[c, j] -= h
            fd = (loss(B, x, xn, up, b, dy, dyn, act) - loss(B, x, xn, dn, b, dy, dyn, act)) / (2 * h)
            assert abs(fd - dw[c, j]) <= 1e-6 * max(1.0, abs(fd)), (c, j, fd, dw[c, j])


@pytest.mark.parametrize("W,B", [(4, 2), (2, 4), (5, 1)])
def test_adjoint_identity(W, B):
    T, C = CU[-1], 4
    x, xn, w, _, dy, dyn = draw(200 + W, T, C, W, bias=False)
    y, yn = oracle.shortconv_dual(CU, PROMPTS, B, x, xn, w)
    dx, dxn, dw, db = oracle.shortconv_dual_bwd(CU, PROMPTS, B, x, xn, w, dy, dyn)
    lhs = np.sum(dy * y) + np.sum(dyn * yn)
    assert abs(lhs - (np.sum(dx * x) + np.sum(dxn * xn))) <= 1e-11 * max(1.0, abs(lhs))
    assert abs(lhs - np.sum(dw * w)) <= 1e-11 * max(1.0, abs(lhs))
    # with no bias the bias gradient is still the sum of the output gradients
    want_db = dy.sum(axis=0) + sum(dyn[CU[i] + PROMPTS[i]:CU[i + 1]].sum(axis=0) for i in range(len(PROMPTS)))
    assert np.allclose(db, want_db, rtol=1e-12, atol=1e-12)


def test_one_hot_output_gradient_returns_the_taps():
    W, B, C = 4, 2, 2
    T = CU[-1]
    rng = np.random.default_rng(5)
    x, xn = rng.standard_normal((T, C)), rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    z = np.zeros((T, C))
    # clean output at doc 4 (starts at 20, prompt 8), local position 2: taps at
    # local positions -1..2, the one before the document start reads nothing
    t, c = 22, 1
    dy = z.copy(); dy[t, c] = 1.0
    dx, dxn, dw, _ = oracle.shortconv_dual_bwd(CU, PROMPTS, B, x, xn, w, dy, z)
    want = np.zeros((T, C)); want_w = np.zeros((C, W))
    for j in range(W):
        m = t - (W - 1) + j
        if m >= 20:
            want[m, c] = w[c, j]
            want_w[c, j] = x[m, c]
    assert np.array_equal(dx, want) and not dxn.any() and np.array_equal(dw, want_w)
    # noisy output of doc 3 (starts at 11, no prompt, B = 2) at local 5: its
    # block starts at local 4, so taps at local 4, 5 read x~ and 2, 3 read x
    t = 16
    dyn = z.copy(); dyn[t, c] = 1.0
    dx, dxn, dw, _ = oracle.shortconv_dual_bwd(CU, PROMPTS, B, x, xn, w, z, dyn)
    wx, wxn, ww = np.zeros((T, C)), np.zeros((T, C)), np.zeros((C, W))
    for j in range(W):
        m = t - (W - 1) + j
        if m >= 15:
            wxn[m, c] = w[c, j]; ww[c, j] = xn[m, c]
        else:
            wx[m, c] = w[c, j]; ww[c, j] = x[m, c]
    assert np.array_equal(dx, wx) and np.array_equal(dxn, wxn) and np.array_equal(dw, ww)


def test_structure_prompt_rows_and_documents():
    W, B, C = 3, 2, 3
    T = CU[-1]
    x, xn, w, b, dy, dyn = draw(9, T, C, W)
    dx, dxn, dw, db = oracle.shortconv_dual_bwd(CU, PROMPTS, B, x, xn, w, dy, dyn, bias=b, activation=1)
    for i, p in enumerate(PROMPTS):
        assert not dxn[CU[i]:CU[i] + p].any()
    # the noisy output gradient's prompt rows are ignored
    dyn2 = dyn.copy()
    for i, p in enumerate(PROMPTS):
        dyn2[CU[i]:CU[i] + p] = 123.0
    r2 = oracle.shortconv_dual_bwd(CU, PROMPTS, B, x, xn, w, dy, dyn2, bias=b, activation=1)
    for a_, b_ in zip((dx, dxn, dw, db), r2):
        assert np.array_equal(a_, b_)
    # an output gradient inside document 3 moves input gradients of document 3 only
    dy3 = np.zeros_like(dy); dy3[11:20] = dy[11:20]
    dyn3 = np.zeros_like(dyn); dyn3[11:20] = dyn[11:20]
    g3 = oracle.shortconv_dual_bwd(CU, PROMPTS, B, x, xn, w, dy3, dyn3, bias=b, activation=1)
    outside = np.r_[0:11, 20:T]
    assert not g3[0][outside].any() and not g3[1][outside].any()
