"""Pin of the oracle's serving step with the ShortConv in front
(oracle.block_step_conv, oracle.conv_cache_fill) against the training-path
definition: serving one document incrementally -- prefill the prompt into a
pool slot and a clean-history cache, then for every block an EVAL of the noisy
block followed by a COMMIT of the clean block -- gives exactly the outputs
of the whole-document prologue (ShortConv, SiLU, q/k L2 norm) followed by the
dual GDN forward: every noisy block's outputs, every clean output, and the
final state.  Prompts longer than, shorter than and equal to zero relative
to the conv history are covered.
"""
import numpy as np
import pytest

import oracle

H, D, B, W = 2, 4, 4, 4


@pytest.mark.parametrize("P,act", [(8, 0), (2, 1), (0, 1)])
def test_incremental_serving_equals_full_forward(P, act):
    n_blocks = 3
    n = P + n_blocks * B
    C = H * D
    rng = np.random.default_rng(70 + P)
    xs = [rng.standard_normal((n, C)) for _ in range(3)]
    xns = [rng.standard_normal((n, C)) for _ in range(3)]
    ws = [rng.uniform(-0.6, 0.6, (C, W)) for _ in range(3)]
    a, b = rng.uniform(0.8, 1.0, (n, H)), rng.uniform(0.1, 0.9, (n, H))
    an, bn = rng.uniform(0.8, 1.0, (n, H)), rng.uniform(0.1, 0.9, (n, H))
    heads = lambda y: y.reshape(-1, H, D)

    ys, yns = oracle.qkv_prologue([0, n], [P], B, D, xs, xns, ws, activation=act)
    o, on, hf = oracle.gdn_dual_fwd([0, n], [P], *map(heads, ys), a, b, *map(heads, yns), an, bn, B)

    n_slots, slot = 3, 1
    pool = np.zeros((n_slots, H, D, D))
    cache = np.zeros((n_slots, W - 1, 3, C))
    if P > 0:
        yp, ynp = oracle.qkv_prologue([0, P], [P], B, D, [x[:P] for x in xs], [x[:P] for x in xns], ws,
                                      activation=act)
        _, _, hp = oracle.gdn_dual_fwd([0, P], [P], *map(heads, yp), a[:P], b[:P], *map(heads, ynp), an[:P],
                                       bn[:P], B)
        pool[slot] = hp[0]
        oracle.conv_cache_fill([0, P], [x[:P] for x in xs], W, [slot], cache)
    for blk in range(n_blocks):
        rows = slice(P + blk * B, P + (blk + 1) * B)
        req = lambda arr: arr[rows][None]
        oe = oracle.block_step_conv([slot], pool, cache, D, [req(x) for x in xns], ws, req(an), req(bn),
                                    oracle.EVAL, activation=act)
        np.testing.assert_allclose(oe[0], on[rows], rtol=1e-11, atol=1e-12)
        oc = oracle.block_step_conv([slot], pool, cache, D, [req(x) for x in xs], ws, req(a), req(b),
                                    oracle.COMMIT, activation=act)
        np.testing.assert_allclose(oc[0], o[rows], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(pool[slot], hf[0], rtol=1e-11, atol=1e-12)
    # the other slots were never touched
    assert not pool[[0, 2]].any() and not cache[[0, 2]].any()
