"""GPU parity of flare_gdn_block_step and flare_shortconv_dual against the fp64
oracle, through the C ABI."""
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


def _block_dev(blk, dev, bf16=True):
    q, k, v, a, b = blk
    return (to_dev(q, dev, bf16), to_dev(k, dev, bf16), to_dev(v, dev, bf16), to_dev(a, dev), to_dev(b, dev))


def test_serving_cycle_full_size(g, dev):
    """256 requests x 16 heads, fp32 128x128 states, B=4: four EVALs then a
    COMMIT; the pool is bit-identical after every EVAL."""
    import torch
    s = wl.serving()
    pool = to_dev(s.pool, dev)
    slot = to_dev(s.slot_idx, dev)
    ref_pool = s.pool.astype(np.float64)
    before = pool.clone()
    for e, blk in enumerate(s.evals):
        o = g.block_step(slot, pool, *_block_dev(blk, dev), g.EVAL, slot_idx_host=s.slot_idx)
        torch.cuda.synchronize()
        ro = oracle.block_step(s.slot_idx, ref_pool, *blk, oracle.EVAL)
        err = rel_rms(to_np(o), ro)
        print("eval", e, err)
        assert err <= TOL_BF16
        assert torch.equal(pool, before), "EVAL must not write the pool"
    o = g.block_step(slot, pool, *_block_dev(s.commit, dev), g.COMMIT, slot_idx_host=s.slot_idx)
    torch.cuda.synchronize()
    ro = oracle.block_step(s.slot_idx, ref_pool, *s.commit, oracle.COMMIT)
    err_o = rel_rms(to_np(o), ro)
    got_pool = to_np(pool)
    err_s = rel_rms(got_pool[s.slot_idx], ref_pool[s.slot_idx])
    print("commit", err_o, err_s)
    assert err_o <= TOL_BF16 and err_s <= 1e-5
    untouched = np.setdiff1d(np.arange(s.pool.shape[0]), s.slot_idx)
    assert np.array_equal(got_pool[untouched], s.pool[untouched].astype(np.float64))


def test_eval_repeatable_and_commit_without_outputs(g, dev):
    import torch
    s = wl.serving(seed=41, n_req=7, H=3, n_slots=11, n_evals=1)
    pool = to_dev(s.pool, dev)
    slot = to_dev(s.slot_idx, dev)
    o1 = g.block_step(slot, pool, *_block_dev(s.evals[0], dev), g.EVAL)
    o2 = g.block_step(slot, pool, *_block_dev(s.evals[0], dev), g.EVAL)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    g.block_step(slot, pool, *_block_dev(s.commit, dev), g.COMMIT, o=False)
    torch.cuda.synchronize()
    ref_pool = s.pool.astype(np.float64)
    oracle.block_step(s.slot_idx, ref_pool, *s.commit, oracle.COMMIT)
    assert rel_rms(to_np(pool), ref_pool) <= 1e-5


@pytest.mark.parametrize("B,d,io", [(1, 128, "bf16"), (8, 128, "bf16"), (16, 128, "bf16"), (32, 128, "bf16"),
                                    (4, 16, "f32"), (16, 16, "f32"), (16, 128, "f32"), (32, 128, "f32")])
def test_block_step_sizes(g, dev, B, d, io):
    import torch
    rng = np.random.default_rng(42 + B + d)
    R, H, n_slots = 5, 2, 9
    slot = rng.permutation(n_slots)[:R].astype(np.int32)
    pool = (rng.standard_normal((n_slots, H, d, d)) / np.sqrt(d)).astype(np.float32)
    rnd = wl.round_bf16 if io == "bf16" else (lambda x: x.astype(np.float32))
    nrm = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    blk = (rnd(nrm(rng.standard_normal((R, B, H, d))).astype(np.float32)),
           rnd(nrm(rng.standard_normal((R, B, H, d))).astype(np.float32)),
           rnd(rng.standard_normal((R, B, H, d)).astype(np.float32)),
           rng.uniform(0.8, 1.0, (R, B, H)).astype(np.float32),
           rng.uniform(0.0, 1.0, (R, B, H)).astype(np.float32))
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    for mode in (g.EVAL, g.COMMIT):
        p = to_dev(pool, dev)
        o = g.block_step(to_dev(slot, dev), p, *_block_dev(blk, dev, io == "bf16"), mode)
        torch.cuda.synchronize()
        rp = pool.astype(np.float64)
        ro = oracle.block_step(slot, rp, *blk, mode)
        assert rel_rms(to_np(o), ro) <= tol, (mode, rel_rms(to_np(o), ro))
        assert rel_rms(to_np(p), rp) <= 1e-5


# ------------------------------------------------------------------ ShortConv

@pytest.mark.parametrize("W", [1, 2, 4, 5, 8])
def test_shortconv_position_tags_exact(g, dev, W):
    """fp32 x[t] = doc*1000 + t, x~ = -x - 1, one-hot weights: every tap's
    source and position is read back exactly (documents across the 64-token
    runs and 256-token blocks of the kernel, one shorter than the window)."""
    import torch
    lens, prompts, B, C = [37, 8, 0, 51, 3, 230], [12, 0, 0, 4, 0, 100], 4, 8
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(L) + 1000 * i for i, L in enumerate(lens)]).astype(np.float32)
    x = np.repeat(pos[:, None], C, axis=1)
    xn = -x - 1
    vl = g.Varlen(cu, prompts, dev)
    for lag in range(W):
        w = np.zeros((C, W), np.float32)
        w[:, W - 1 - lag] = 1.0
        y, yn = g.shortconv_dual(vl, B, to_dev(x, dev), to_dev(xn, dev), to_dev(w, dev))
        torch.cuda.synchronize()
        ry, ryn = oracle.shortconv_dual(cu, prompts, B, x, xn, w)
        np.testing.assert_array_equal(to_np(y), ry)
        np.testing.assert_array_equal(to_np(yn), ryn)


@pytest.mark.parametrize("W,act,bias", [(4, 0, False), (3, 1, True), (8, 0, True), (1, 1, False)])
def test_shortconv_bf16_small(g, dev, W, act, bias):
    import torch
    rng = np.random.default_rng(50 + W)
    lens, prompts, B, C = [70, 5, 129], [20, 4, 64], 4, 48
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = wl.round_bf16(rng.standard_normal((T, C)).astype(np.float32))
    xn = wl.round_bf16(rng.standard_normal((T, C)).astype(np.float32))
    w = rng.uniform(-0.5, 0.5, (C, W)).astype(np.float32)
    bb = rng.standard_normal(C).astype(np.float32) if bias else None
    vl = g.Varlen(cu, prompts, dev)
    y, yn = g.shortconv_dual(vl, B, to_dev(x, dev, True), to_dev(xn, dev, True), to_dev(w, dev),
                             bias=to_dev(bb, dev) if bias else None, activation=act)
    torch.cuda.synchronize()
    ry, ryn = oracle.shortconv_dual(cu, prompts, B, x, xn, w, bias=bb, activation=act)
    assert rel_rms(to_np(y), ry) <= TOL_BF16
    assert rel_rms(to_np(yn), ryn) <= TOL_BF16
    for i in range(3):
        assert not np.any(to_np(yn)[cu[i]:cu[i] + prompts[i]])


def test_shortconv_packed_full_size_sampled_channels(g, dev):
    """One packed row of 32768 tokens, 8 Dirichlet-split docs, 3*32*128 channels,
    W=4, bf16; the oracle checks 512 sampled channels."""
    import torch
    p = wl.packed_conv()
    vl = g.Varlen(p["cu_seqlens"], p["prompt_lens"], dev)
    y, yn = g.shortconv_dual(vl, p["block_size"], to_dev(p["x"], dev, True), to_dev(p["xn"], dev, True),
                             to_dev(p["weight"], dev))
    torch.cuda.synchronize()
    ch = np.r_[0:256, p["x"].shape[1] - 256:p["x"].shape[1]]
    ry, ryn = oracle.shortconv_dual(p["cu_seqlens"], p["prompt_lens"], p["block_size"],
                                    p["x"][:, ch], p["xn"][:, ch], p["weight"][ch])
    assert rel_rms(to_np(y[:, ch]), ry) <= TOL_BF16
    assert rel_rms(to_np(yn[:, ch]), ryn) <= TOL_BF16
