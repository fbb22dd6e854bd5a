"""Pins of the oracle's AR-Trust verify and scatter (oracle.gdn_verify,
oracle.gdn_scatter, and the replay form oracle.gdn_commit_prefix), against
the other oracle paths they must agree with:
  * every candidate state equals the dual forward's final state over a
    one-document batch of the first t+1 drafted tokens (all clean), started
    from the pool state -- the forward's own document loop, not the step code;
  * the verify outputs equal the forward's clean outputs over the same tokens;
  * verify never writes the pool and is repeatable;
  * scatter(r) followed by a COMMIT of the remaining K - r tokens leaves the
    pool exactly where a COMMIT of all K tokens would (the rollback is a true
    prefix); r = 0 leaves the slot, r = K is the last candidate; counts
    outside [0, K] are clamped.
"""
import numpy as np
import pytest

import oracle


def draw(seed, R, K, H, dk, dv, n_slots):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((R, K, H, dk))
    k = rng.standard_normal((R, K, H, dk))
    k /= np.linalg.norm(k, axis=3, keepdims=True)
    v = rng.standard_normal((R, K, H, dv))
    a = rng.uniform(0.8, 1.0, (R, K, H))
    b = rng.uniform(0.1, 0.9, (R, K, H))
    pool = rng.standard_normal((n_slots, H, dk, dv))
    slots = rng.permutation(n_slots)[:R].astype(np.int32)
    return slots, pool, q, k, v, a, b


def test_candidates_are_prefix_forward_states():
    R, K, H, dk, dv = 3, 5, 2, 4, 3
    slots, pool, q, k, v, a, b = draw(1, R, K, H, dk, dv, 7)
    before = pool.copy()
    o, cand = oracle.gdn_verify(slots, pool, q, k, v, a, b)
    np.testing.assert_array_equal(pool, before)
    for r in range(R):
        h0 = pool[slots[r]][None]
        for t in range(K):
            n = t + 1
            xs = [x[r, :n] for x in (q, k, v, a, b)]
            # one document of n clean tokens (prompt = whole document): no noisy part
            fo, _, hf = oracle.gdn_dual_fwd([0, n], [n], *xs, *xs, 1, h0=h0)
            np.testing.assert_allclose(cand[r, t], hf[0], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(o[r, t], fo[t], rtol=1e-12, atol=1e-12)
    o2, cand2 = oracle.gdn_verify(slots, pool, q, k, v, a, b)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(cand, cand2)


@pytest.mark.parametrize("accepted", [[0, 3, 5, 1], [5, 5, 0, 2], [-2, 9, 4, 0]])
def test_scatter_then_commit_rest_equals_commit_all(accepted):
    R, K, H, dk, dv = 4, 5, 2, 3, 4
    slots, pool, q, k, v, a, b = draw(2, R, K, H, dk, dv, 9)
    o, cand = oracle.gdn_verify(slots, pool, q, k, v, a, b)
    full = pool.copy()
    oracle.block_step(slots, full, q, k, v, a, b, oracle.COMMIT)
    rolled = pool.copy()
    oracle.gdn_scatter(slots, accepted, cand, rolled)
    untouched = [s for s in range(pool.shape[0]) if s not in slots]
    np.testing.assert_array_equal(rolled[untouched], pool[untouched])
    for i in range(R):
        r = min(max(accepted[i], 0), K)
        if r == 0:
            np.testing.assert_array_equal(rolled[slots[i]], pool[slots[i]])
        else:
            np.testing.assert_array_equal(rolled[slots[i]], cand[i, r - 1])
        if r < K:
            rest = [x[i:i + 1, r:] for x in (q, k, v, a, b)]
            oracle.block_step(slots[i:i + 1], rolled, *rest, oracle.COMMIT)
        np.testing.assert_allclose(rolled[slots[i]], full[slots[i]], rtol=1e-12, atol=1e-12)


def test_verify_rejects_duplicate_slots():
    x = np.zeros((2, 2, 1, 2))
    g = np.ones((2, 2, 1))
    with pytest.raises(ValueError):
        oracle.gdn_verify([1, 1], np.zeros((3, 1, 2, 2)), x, x, x, g, g)


def test_commit_prefix_equals_verify_then_scatter():
    """The replay form of the rollback (oracle.gdn_commit_prefix: the step's
    COMMIT over the first r tokens) lands every slot where the candidate form
    (oracle.gdn_verify's token-by-token candidates, then oracle.gdn_scatter)
    does, for r = 0, 1..K and out-of-range counts; its outputs are verify's
    outputs on the replayed tokens and zero past them; other slots untouched."""
    R, K, H, dk, dv = 6, 4, 2, 4, 3
    slots, pool, q, k, v, a, b = draw(5, R, K, H, dk, dv, 9)
    accepted = [0, 1, 2, K, -2, K + 3]
    o_ver, cand = oracle.gdn_verify(slots, pool, q, k, v, a, b)
    via_scatter = oracle.gdn_scatter(slots, accepted, cand, pool.copy())
    via_replay = pool.copy()
    o = oracle.gdn_commit_prefix(slots, via_replay, q, k, v, a, b, accepted)
    np.testing.assert_allclose(via_replay, via_scatter, rtol=1e-12, atol=1e-12)
    for i in range(R):
        r = min(max(accepted[i], 0), K)
        np.testing.assert_allclose(o[i, :r], o_ver[i, :r], rtol=1e-12, atol=1e-12)
        assert not o[i, r:].any()
        if r == 0:
            np.testing.assert_array_equal(via_replay[slots[i]], pool[slots[i]])
    others = np.setdiff1d(np.arange(pool.shape[0]), slots)
    np.testing.assert_array_equal(via_replay[others], pool[others])
