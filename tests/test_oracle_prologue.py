"""Pins of the oracle's QKV prologue (ShortConv -> optional SiLU -> per-head L2
norm of q and k) and its reverse mode, against things fixed independently of
its numpy code:
  * composition with the oracle's C forward: the dual GDN forward on the
    prologue's outputs (no flag) equals the C forward on the raw ShortConv
    outputs with its own q/k L2 flag (an independent implementation of the
    normalisation, including its epsilon);
  * the same composition for the reverse mode: the prologue's reverse mode
    applied to the GDN gradients w.r.t. the normalised q, k equals the plain
    ShortConv reverse mode applied to the C backward's gradients w.r.t. the
    raw q, k under the L2 flag;
  * central finite differences of <dy, y> + <dy~, y~> summed over q, k, v for
    every input, with and without SiLU;
  * structure: v passes through the ShortConv alone, q/k rows have unit norm,
    noisy prompt rows are zero.
"""
import numpy as np
import pytest

import oracle

CU = [0, 11, 11, 20, 30, 36]
PROMPTS = [4, 0, 0, 8, 4]
H, D = 2, 4
T = CU[-1]


def draw(seed, W):
    rng = np.random.default_rng(seed)
    xs = [rng.standard_normal((T, H * D)) for _ in range(3)]
    xns = [rng.standard_normal((T, H * D)) for _ in range(3)]
    ws = [rng.uniform(-0.7, 0.7, (H * D, W)) for _ in range(3)]
    return xs, xns, ws


def gates(seed):
    rng = np.random.default_rng(seed)
    a = np.exp(-0.1 * np.log1p(np.exp(rng.standard_normal((T, H)))))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    an = np.exp(-0.1 * np.log1p(np.exp(rng.standard_normal((T, H)))))
    bn = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return a, b, an, bn


def heads(y):
    return y.reshape(T, H, D)


@pytest.mark.parametrize("act,B", [(0, 2), (1, 4)])
def test_forward_matches_the_c_l2_flag(act, B):
    xs, xns, ws = draw(11 + act, 3)
    ys, yns = oracle.qkv_prologue(CU, PROMPTS, B, D, xs, xns, ws, activation=act)
    raw, rawn = oracle.qkv_prologue(CU, PROMPTS, B, D, xs, xns, ws, activation=act, l2=False)
    a, b, an, bn = gates(5)
    o1, on1, h1 = oracle.gdn_dual_fwd(CU, PROMPTS, *map(heads, ys), a, b, *map(heads, yns), an, bn, B)
    o2, on2, h2 = oracle.gdn_dual_fwd(CU, PROMPTS, *map(heads, raw), a, b, *map(heads, rawn), an, bn, B,
                                      flags=oracle.FLAG_QK_L2NORM)
    for u, v in ((o1, o2), (on1, on2), (h1, h2)):
        assert np.allclose(u, v, rtol=1e-12, atol=1e-12)


def test_structure():
    xs, xns, ws = draw(3, 4)
    ys, yns = oracle.qkv_prologue(CU, PROMPTS, 4, D, xs, xns, ws, activation=1)
    raw, rawn = oracle.qkv_prologue(CU, PROMPTS, 4, D, xs, xns, ws, activation=1, l2=False)
    assert np.array_equal(ys[2], raw[2]) and np.array_equal(yns[2], rawn[2])
    for sec in range(2):
        n = np.linalg.norm(heads(ys[sec]), axis=2)
        big = np.linalg.norm(heads(raw[sec]), axis=2) > 0.1
        assert np.allclose(n[big], 1.0, atol=1e-4)
    for i, p in enumerate(PROMPTS):
        for sec in range(3):
            assert not yns[sec][CU[i]:CU[i] + p].any()


@pytest.mark.parametrize("act", [0, 1])
def test_finite_differences(act):
    B, W = 2, 3
    xs, xns, ws = draw(21 + act, W)
    rng = np.random.default_rng(8)
    dys = [rng.standard_normal((T, H * D)) for _ in range(3)]
    dyns = [rng.standard_normal((T, H * D)) for _ in range(3)]
    dxs, dxns, dws = oracle.qkv_prologue_bwd(CU, PROMPTS, B, D, xs, xns, ws, dys, dyns, activation=act)

    def loss(xs_, xns_, ws_):
        ys, yns = oracle.qkv_prologue(CU, PROMPTS, B, D, xs_, xns_, ws_, activation=act)
        return sum(float(np.sum(dys[s] * ys[s]) + np.sum(dyns[s] * yns[s])) for s in range(3))

    h = 1e-6
    for which, grads in (("x", dxs), ("xn", dxns), ("w", dws)):
        for sec in range(3):
            base = {"x": xs, "xn": xns, "w": ws}[which]
            d = rng.standard_normal(base[sec].shape)
            up = [u.copy() for u in base]
            dn = [u.copy() for u in base]
            up[sec] += h * d
            dn[sec] -= h * d
            args_up = {"x": xs, "xn": xns, "w": ws}
            args_dn = dict(args_up)
            args_up = dict(args_up, **{which: up})
            args_dn = dict(args_dn, **{which: dn})
            fd = (loss(args_up["x"], args_up["xn"], args_up["w"]) - loss(args_dn["x"], args_dn["xn"], args_dn["w"])) / (2 * h)
            an = float(np.sum(grads[sec] * d))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (which, sec, fd, an)


@pytest.mark.parametrize("act,B", [(0, 4), (1, 2)])
def test_reverse_matches_the_c_l2_flag(act, B):
    xs, xns, ws = draw(31 + act, 3)
    ys, yns = oracle.qkv_prologue(CU, PROMPTS, B, D, xs, xns, ws, activation=act)
    raw, rawn = oracle.qkv_prologue(CU, PROMPTS, B, D, xs, xns, ws, activation=act, l2=False)
    a, b, an, bn = gates(6)
    rng = np.random.default_rng(9)
    do = rng.standard_normal((T, H, D))
    don = rng.standard_normal((T, H, D))
    g1 = oracle.gdn_dual_bwd(CU, PROMPTS, *map(heads, ys), a, b, *map(heads, yns), an, bn, B, do, don)
    g2 = oracle.gdn_dual_bwd(CU, PROMPTS, *map(heads, raw), a, b, *map(heads, rawn), an, bn, B, do, don,
                             flags=oracle.FLAG_QK_L2NORM)
    flat = lambda x: x.reshape(T, H * D)
    r1 = oracle.qkv_prologue_bwd(CU, PROMPTS, B, D, xs, xns, ws, [flat(g1[k]) for k in ("dq", "dk", "dv")],
                                 [flat(g1[k]) for k in ("dqn", "dkn", "dvn")], activation=act)
    r2 = oracle.qkv_prologue_bwd(CU, PROMPTS, B, D, xs, xns, ws, [flat(g2[k]) for k in ("dq", "dk", "dv")],
                                 [flat(g2[k]) for k in ("dqn", "dkn", "dvn")], activation=act, l2=False)
    for lst1, lst2 in zip(r1, r2):
        for u, v in zip(lst1, lst2):
            assert np.allclose(u, v, rtol=1e-10, atol=1e-10)
