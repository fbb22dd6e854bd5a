"""GPU parity of the serving step with the ShortConv in front
(flare_gdn_block_step_conv, flare_conv_cache_fill) through the C-ABI binding,
against the fp64 oracle (oracle.block_step_conv, oracle.conv_cache_fill):
  * EVAL and COMMIT from random pools and clean histories, widths 1 to 8
    (both LDS sizings: up to 4 and up to 8),
    blocks of 4 and 8, fp32 (d = 16) and bf16 (d = 128) io, with and without
    SiLU; EVAL leaves the pool and the history cache bit-identical, COMMIT's
    new history is the exact last W-1 raw rows;
  * serving documents end to end on the GPU -- the prologue and the dual
    forward prefill the prompts straight into pool slots, the history cache is
    filled, then every block is drafted (EVAL) and fixed (COMMIT) -- against
    the oracle's same sequence (whose equality with the whole-document
    forward is pinned in the CPU tests).
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


def _round(x, bf16):
    return wl.round_bf16(np.asarray(x, np.float32)) if bf16 else np.asarray(x, np.float32)


@pytest.mark.parametrize("d,io,W,B,act", [(16, "f32", 4, 4, 0), (16, "f32", 1, 8, 1), (128, "bf16", 4, 4, 1),
                                          (128, "bf16", 8, 8, 0), (128, "bf16", 4, 8, 1), (16, "f32", 5, 4, 1),
                                          (128, "bf16", 3, 8, 0), (128, "bf16", 2, 4, 1), (128, "bf16", 6, 4, 1)])
def test_block_step_conv_modes(g, dev, d, io, W, B, act):
    import torch
    bf16 = io == "bf16"
    R, H, n_slots = 5, 2, 8
    C = H * d
    rng = np.random.default_rng(80 + d + W + B)
    slots = rng.permutation(n_slots)[:R].astype(np.int32)
    pool = (rng.standard_normal((n_slots, H, d, d)) / np.sqrt(d)).astype(np.float32)
    cache = _round(rng.standard_normal((n_slots, W - 1, 3, C)), bf16)
    ws = [rng.uniform(-0.6, 0.6, (C, W)).astype(np.float32) for _ in range(3)]
    for mode in (oracle.EVAL, oracle.COMMIT):
        xs = [_round(rng.standard_normal((R, B, C)), bf16) for _ in range(3)]
        a = rng.uniform(0.85, 1.0, (R, B, H)).astype(np.float32)
        b = rng.uniform(0.1, 0.9, (R, B, H)).astype(np.float32)
        gpool = to_dev(pool, dev)
        gcache = to_dev(cache, dev, bf16) if W > 1 else None
        before_pool = gpool.clone()
        before_cache = gcache.clone() if W > 1 else None
        o = g.block_step_conv(to_dev(slots, dev), gpool, gcache, [to_dev(w, dev) for w in ws],
                              *(to_dev(x.reshape(R, B, H, d), dev, bf16) for x in xs), to_dev(a, dev), to_dev(b, dev),
                              g.EVAL if mode == oracle.EVAL else g.COMMIT, activation=act, slot_idx_host=slots)
        torch.cuda.synchronize()
        rpool, rcache = pool.astype(np.float64), cache.astype(np.float64)
        ro = oracle.block_step_conv(slots, rpool, rcache, d, xs, ws, a, b, mode, activation=act)
        assert rel_rms(to_np(o), ro) <= (TOL_BF16 if bf16 else TOL_F32), mode
        if mode == oracle.EVAL:
            assert torch.equal(gpool, before_pool)
            if W > 1:
                assert torch.equal(gcache, before_cache)
        else:
            got = gpool.cpu().numpy()
            assert rel_rms(got[slots], rpool[slots]) <= TOL_F32
            others = np.setdiff1d(np.arange(n_slots), slots)
            assert np.array_equal(got[others], pool[others])
            if W > 1:
                assert np.array_equal(to_np(gcache), rcache)


@pytest.mark.parametrize("d,io", [(16, "f32"), (128, "bf16")])
def test_serving_documents_end_to_end(g, dev, d, io):
    import torch
    bf16 = io == "bf16"
    H, B, W, act = 2, 4, 4, 1
    C = H * d
    prompts = [8, 0, 12]  # an empty prompt: all history rows are zero
    n_blocks = 3
    R = len(prompts)
    n_slots = 6
    rng = np.random.default_rng(90 + d)
    slots = np.array([4, 0, 2], np.int32)
    ws = [rng.uniform(-0.6, 0.6, (C, W)).astype(np.float32) for _ in range(3)]
    # prompts packed as one batch of documents (all clean)
    cu = np.concatenate([[0], np.cumsum(prompts)]).astype(np.int32)
    T = int(cu[-1])
    xp = [_round(rng.standard_normal((T, C)), bf16) for _ in range(3)]
    ga = rng.uniform(0.85, 1.0, (T, H)).astype(np.float32)
    gb = rng.uniform(0.1, 0.9, (T, H)).astype(np.float32)
    # GPU prefill: prologue -> forward into the pool slots -> history cache
    vl = g.Varlen(cu, prompts, dev)
    up = lambda x: to_dev(x, dev, bf16)
    ys, yns = g.qkv_prologue(vl, B, d, [up(x) for x in xp], [up(x) for x in xp], [to_dev(w, dev) for w in ws],
                             activation=act)
    gpool = to_dev(np.zeros((n_slots, H, d, d), np.float32), dev)
    gslots = to_dev(slots, dev)
    hv = lambda t: t.view(T, H, d)
    g.gdn_dual_fwd_pool(vl, hv(ys[0]), hv(ys[1]), hv(ys[2]), to_dev(ga, dev), to_dev(gb, dev), hv(yns[0]),
                        hv(yns[1]), hv(yns[2]), to_dev(ga, dev), to_dev(gb, dev), B, gslots, gpool,
                        doc_slot_host=slots)
    gcache = torch.zeros((n_slots, W - 1, 3, C), dtype=torch.bfloat16 if bf16 else torch.float32, device=dev)
    g.conv_cache_fill(vl, d, W, [up(x) for x in xp], gslots, gcache, doc_slot_host=slots)
    # oracle prefill: the same steps, its prologue outputs rounded where the GPU stores io
    rys, ryns = oracle.qkv_prologue(cu, prompts, B, d, xp, xp, ws, activation=act)
    rys, ryns = [_round(y, bf16).astype(np.float64) for y in rys], [_round(y, bf16).astype(np.float64) for y in ryns]
    rh = lambda y: y.reshape(T, H, d)
    _, _, hf = oracle.gdn_dual_fwd(cu, prompts, *map(rh, rys), ga, gb, *map(rh, ryns), ga, gb, B)
    rpool = np.zeros((n_slots, H, d, d))
    rpool[slots] = hf
    rcache = oracle.conv_cache_fill(cu, xp, W, slots, np.zeros((n_slots, W - 1, 3, C)))
    torch.cuda.synchronize()
    # bf16: an intermediate q/k/v value next to a rounding boundary may round the
    # other way on the two sides, so the states agree to 1e-3 rather than 1e-4
    state_tol = 1e-3 if bf16 else TOL_F32
    assert rel_rms(gpool.cpu().numpy()[slots], rpool[slots]) <= state_tol
    assert np.array_equal(to_np(gcache), rcache)
    # decode: draft (EVAL) then fix (COMMIT) every block
    for blk in range(n_blocks):
        for mode in (oracle.EVAL, oracle.COMMIT):
            xs = [_round(rng.standard_normal((R, B, C)), bf16) for _ in range(3)]
            a = rng.uniform(0.85, 1.0, (R, B, H)).astype(np.float32)
            b = rng.uniform(0.1, 0.9, (R, B, H)).astype(np.float32)
            o = g.block_step_conv(gslots, gpool, gcache, [to_dev(w, dev) for w in ws],
                                  *(up(x.reshape(R, B, H, d)) for x in xs), to_dev(a, dev), to_dev(b, dev),
                                  g.EVAL if mode == oracle.EVAL else g.COMMIT, activation=act, slot_idx_host=slots)
            ro = oracle.block_step_conv(slots, rpool, rcache, d, xs, ws, a, b, mode, activation=act)
            torch.cuda.synchronize()
            assert rel_rms(to_np(o), ro) <= (TOL_BF16 if bf16 else TOL_F32), (blk, mode)
    assert rel_rms(gpool.cpu().numpy()[slots], rpool[slots]) <= state_tol
    assert np.array_equal(to_np(gcache), rcache)
