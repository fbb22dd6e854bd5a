"""Pins for the oracle's reverse mode: central finite differences of the oracle
forward (itself pinned by brute force) for every input including the initial
state, plus the structural zeros the pages imply -- the clean loss does not
reach the noisy inputs, noisy prompt rows carry no gradient, and no gradient
crosses a document boundary ("FLARE: Diffusion for Hybrid Language Model",
papernotes.org notes, Key designs items 2 and 3)."""
import numpy as np
import pytest

import oracle
from test_oracle_pins import rand_case

NAMES = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("a", "dalpha"), ("b", "dbeta"),
         ("qn", "dqn"), ("kn", "dkn"), ("vn", "dvn"), ("an", "dalpha_n"), ("bn", "dbeta_n"),
         ("h0", "dh0")]
ORDER = ("q", "k", "v", "a", "b", "qn", "kn", "vn", "an", "bn")


def loss(c, B, do, don, dhf, flags=0, scale=0.0):
    o, on, hf = oracle.gdn_dual_fwd(c["cu"], c["pl"], *(c[x] for x in ORDER), B, h0=c["h0"],
                                    flags=flags, scale=scale)
    return (o * do).sum() + (on * don).sum() + (hf * dhf).sum()


def grads(c, B, do, don, dhf, flags=0, scale=0.0):
    return oracle.gdn_dual_bwd(c["cu"], c["pl"], *(c[x] for x in ORDER), B, do, don,
                               h0=c["h0"], dh_final=dhf, flags=flags, scale=scale)


@pytest.mark.parametrize("flags", [0, oracle.FLAG_QK_L2NORM])
def test_finite_differences_all_inputs(flags):
    rng = np.random.default_rng(40 + flags)
    lens, prompts, B = [7, 6, 5], [2, 0, 5], 2
    H, dk, dv = 2, 3, 2   # dk != dv so a transposed operand cannot pass
    c = rand_case(rng, lens, prompts, H, dk, dv, norm=(flags == 0))
    T = sum(lens)
    do = rng.standard_normal((T, H, dv))
    don = rng.standard_normal((T, H, dv))
    dhf = rng.standard_normal((len(lens), H, dk, dv))
    g = grads(c, B, do, don, dhf, flags=flags, scale=0.7)
    eps = 1e-6
    for name, gname in NAMES:
        x = c[name]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = x[idx]
            x[idx] = orig + eps
            lp = loss(c, B, do, don, dhf, flags, 0.7)
            x[idx] = orig - eps
            lm = loss(c, B, do, don, dhf, flags, 0.7)
            x[idx] = orig
            num[idx] = (lp - lm) / (2 * eps)
        an = g[gname]
        err = np.abs(an - num).max() / max(1.0, np.abs(num).max())
        assert err < 1e-7, (name, err)


def test_structural_zeros():
    rng = np.random.default_rng(50)
    lens, prompts, B = [9, 8], [3, 0], 3
    H, dk, dv = 1, 3, 3
    c = rand_case(rng, lens, prompts, H, dk, dv)
    T = sum(lens)
    do = rng.standard_normal((T, H, dv))
    zero = np.zeros((T, H, dv))
    # clean loss only: noisy inputs get exactly zero gradient
    g = grads(c, B, do, zero, None)
    for key in ("dqn", "dkn", "dvn", "dalpha_n", "dbeta_n"):
        assert not np.any(g[key]), key
    # noisy prompt rows: zero gradient even with a noisy loss
    g = grads(c, B, do, rng.standard_normal((T, H, dv)), None)
    for key in ("dqn", "dkn", "dvn", "dalpha_n", "dbeta_n"):
        assert not np.any(g[key][:3]), key
    # loss on document 0 only: document 1 receives nothing
    do0 = do.copy()
    do0[9:] = 0.0
    don0 = rng.standard_normal((T, H, dv))
    don0[9:] = 0.0
    g = grads(c, B, do0, don0, None)
    for key in ("dq", "dk", "dv", "dalpha", "dbeta", "dqn", "dkn", "dvn", "dalpha_n", "dbeta_n"):
        assert not np.any(g[key][9:]), key
    assert not np.any(g["dh0"][1])


@pytest.mark.parametrize("n,P,B,C", [(40, 8, 4, 16), (37, 12, 4, 8), (64, 0, 8, 32), (20, 20, 4, 8),
                                     (33, 4, 1, 4), (70, 16, 16, 16), (45, 0, 4, 16)])
def test_chunked_backward_algebra_matches(n, P, B, C):
    """The chunk-parallel reverse mode (reverse scan over chunk-start adjoints,
    matrix calculus inside each chunk) that the GPU backward implements equals the
    oracle's token-by-token reverse mode."""
    from brute import chunked_backward
    rng = np.random.default_rng(n + P + B + C)
    c = rand_case(rng, [n], [P], 1, 6, 5)
    do = rng.standard_normal((n, 1, 5))
    don = rng.standard_normal((n, 1, 5))
    dhf = rng.standard_normal((1, 1, 6, 5))
    s = 0.37
    ref = oracle.gdn_dual_bwd(c["cu"], c["pl"], *(c[x] for x in ORDER), B, do, don, h0=c["h0"],
                              dh_final=dhf, scale=s)
    got = chunked_backward(*(c[x][:, 0] for x in ORDER), P, B, c["h0"][0, 0], s, C, do[:, 0], don[:, 0],
                           dhf[0, 0])
    for key, val in got.items():
        r = ref[key][:, 0] if key != "dh0" else ref[key][0, 0]
        err = np.abs(val - r).max() / max(1.0, np.abs(r).max())
        assert err < 1e-11, (key, err)
