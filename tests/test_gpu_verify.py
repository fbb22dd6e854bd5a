"""GPU parity of the AR-Trust pair flare_gdn_verify / flare_gdn_scatter
(through the C-ABI binding) against the fp64 oracle (oracle.gdn_verify,
oracle.gdn_scatter):
  * verify: per-token outputs and the candidate state after every drafted
    token, for K in {4, 8, 16, 32}, d in {16 (fp32 io), 128 (bf16 io)}; the
    pool is bit-identical afterwards;
  * scatter: accepted counts 0, 1..K and out of range (clamped); the accepted
    candidate lands in its slot bit for bit, every other slot (and a slot whose
    count is 0) is bit-identical to before, and the result matches the oracle's
    scatter of its own candidates;
  * the replay pair (flare_gdn_verify_outputs, flare_gdn_commit_prefix):
    causal outputs without candidates, pool untouched; the COMMIT of each
    request's accepted prefix against the oracle's (oracle.gdn_commit_prefix),
    a slot with no accepted token bit-identical, other slots untouched, and
    the slots agree with the GPU's own verify + scatter;
  * the full serving shape: 256 requests x 16 heads, K = 4, d = 128, bf16.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_dual_amd import workloads as wl
from gpu_util import TOL_BF16, TOL_F32, rel_rms, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def g():
    import gated_deltanet_dual_amd as g
    g.lib()
    return g


def draw(seed, R, K, H, d, n_slots, bf16):
    rng = np.random.default_rng(seed)
    rnd = wl.round_bf16 if bf16 else (lambda a: a)
    unit = lambda x: x / np.linalg.norm(x, axis=3, keepdims=True)
    q = rnd(unit(rng.standard_normal((R, K, H, d))).astype(np.float32))
    k = rnd(unit(rng.standard_normal((R, K, H, d))).astype(np.float32))
    v = rnd(rng.standard_normal((R, K, H, d)).astype(np.float32))
    a = rng.uniform(0.85, 1.0, (R, K, H)).astype(np.float32)
    b = rng.uniform(0.1, 0.9, (R, K, H)).astype(np.float32)
    pool = (rng.standard_normal((n_slots, H, d, d)) / np.sqrt(d)).astype(np.float32)
    slots = rng.permutation(n_slots)[:R].astype(np.int32)
    return slots, pool, q, k, v, a, b


def run(g, dev, case, accepted, bf16):
    import torch
    slots, pool, q, k, v, a, b = case
    gpool = to_dev(pool, dev)
    gslot = to_dev(slots, dev)
    before = gpool.clone()
    o, cand = g.gdn_verify(gslot, gpool, to_dev(q, dev, bf16), to_dev(k, dev, bf16), to_dev(v, dev, bf16),
                           to_dev(a, dev), to_dev(b, dev), slot_idx_host=slots)
    torch.cuda.synchronize()
    assert torch.equal(gpool, before), "verify must not write the pool"
    cand_np = cand.cpu().numpy()
    g.gdn_scatter(gslot, to_dev(np.asarray(accepted, np.int32), dev), cand, gpool, slot_idx_host=slots)
    torch.cuda.synchronize()
    return to_np(o), cand_np, gpool.cpu().numpy()


@pytest.mark.parametrize("K,d,bf16", [(4, 16, False), (8, 16, False), (4, 128, True), (8, 128, True),
                                      (16, 128, True), (32, 128, True), (16, 16, False)])
def test_verify_and_scatter_small(g, dev, K, d, bf16):
    R, H, n_slots = 6, 2, 11
    case = draw(10 + K + d, R, K, H, d, n_slots, bf16)
    slots, pool, q, k, v, a, b = case
    accepted = [0, K, 1, K // 2, -3, K + 5]
    o, cand, newpool = run(g, dev, case, accepted, bf16)
    ro, rcand = oracle.gdn_verify(slots, pool.astype(np.float64), q, k, v, a, b)
    assert rel_rms(o, ro) <= (TOL_BF16 if bf16 else TOL_F32)
    assert rel_rms(cand, rcand) <= TOL_F32
    # the copy is exact; untouched slots are bit-identical
    for i, sl in enumerate(slots):
        r = min(max(accepted[i], 0), K)
        if r == 0:
            assert np.array_equal(newpool[sl], pool[sl])
        else:
            assert np.array_equal(newpool[sl], cand[i, r - 1])
    others = np.setdiff1d(np.arange(n_slots), slots)
    assert np.array_equal(newpool[others], pool[others])
    rpool = oracle.gdn_scatter(slots, accepted, rcand, pool.astype(np.float64).copy())
    assert rel_rms(newpool, rpool) <= TOL_F32


def test_verify_and_scatter_full_serving_shape(g, dev):
    """256 requests with distinct slots in a pool of 512 fp32 128 x 128 states,
    16 heads, K = 4 drafted bf16 tokens; the oracle checks every request."""
    s = wl.serving()
    q, k, v, a, b = s.commit
    R, K = q.shape[:2]
    rng = np.random.default_rng(44)
    accepted = rng.integers(0, K + 1, R)
    o, cand, newpool = run(g, dev, (s.slot_idx, s.pool, q, k, v, a, b), accepted, True)
    ro, rcand = oracle.gdn_verify(s.slot_idx, s.pool.astype(np.float64), q, k, v, a, b)
    assert rel_rms(o, ro) <= TOL_BF16
    assert rel_rms(cand, rcand) <= TOL_F32
    rpool = oracle.gdn_scatter(s.slot_idx, accepted, rcand, s.pool.astype(np.float64).copy())
    assert rel_rms(newpool[s.slot_idx], rpool[s.slot_idx]) <= TOL_F32
    others = np.setdiff1d(np.arange(s.pool.shape[0]), s.slot_idx)
    assert np.array_equal(newpool[others], s.pool[others])


@pytest.mark.parametrize("K,d,bf16", [(4, 16, False), (8, 128, True), (32, 128, True)])
def test_replay_pair_small(g, dev, K, d, bf16):
    import torch
    R, H, n_slots = 6, 2, 11
    slots, pool, q, k, v, a, b = draw(30 + K + d, R, K, H, d, n_slots, bf16)
    accepted = np.array([0, K, 1, K // 2, -3, K + 5], np.int32)
    gq, gk, gv = to_dev(q, dev, bf16), to_dev(k, dev, bf16), to_dev(v, dev, bf16)
    ga, gb = to_dev(a, dev), to_dev(b, dev)
    gslot = to_dev(slots, dev)
    gpool = to_dev(pool, dev)
    before = gpool.clone()
    o = g.gdn_verify_outputs(gslot, gpool, gq, gk, gv, ga, gb, slot_idx_host=slots)
    torch.cuda.synchronize()
    assert torch.equal(gpool, before), "the causal read must not write the pool"
    ro, _ = oracle.gdn_verify(slots, pool.astype(np.float64), q, k, v, a, b)
    tol = TOL_BF16 if bf16 else TOL_F32
    assert rel_rms(to_np(o), ro) <= tol
    # the prefix commit, with its outputs
    op = torch.zeros_like(o)
    g.gdn_commit_prefix(gslot, gpool, gq, gk, gv, ga, gb, to_dev(accepted, dev), slot_idx_host=slots, o=op)
    torch.cuda.synchronize()
    got = gpool.cpu().numpy()
    rpool = pool.astype(np.float64).copy()
    rop = oracle.gdn_commit_prefix(slots, rpool, q, k, v, a, b, accepted)
    assert rel_rms(got[slots], rpool[slots]) <= TOL_F32
    assert rel_rms(to_np(op), rop) <= tol
    for i, sl in enumerate(slots):
        r = min(max(int(accepted[i]), 0), K)
        if r == 0:
            assert np.array_equal(got[sl], pool[sl])
        assert not to_np(op)[i, r:].any(), "rows past the accepted prefix are not written"
    others = np.setdiff1d(np.arange(n_slots), slots)
    assert np.array_equal(got[others], pool[others])
    # the same slots as the candidate route on the GPU
    _, _, via_scatter = run(g, dev, (slots, pool, q, k, v, a, b), accepted, bf16)
    assert rel_rms(got[slots], via_scatter[slots]) <= TOL_F32
