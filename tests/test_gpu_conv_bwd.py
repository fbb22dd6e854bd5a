"""GPU parity of flare_shortconv_dual_bwd (through the C-ABI binding) against
the fp64 oracle's reverse mode (oracle.shortconv_dual_bwd) on the same seeded
inputs.

  * exact: small-integer inputs, weights and output gradients (fp32 and bf16
    io), so every sum is exact and any misplaced tap, source or document boundary shows as a
    nonzero difference;
  * ragged documents (empty, shorter than the window, across the 64-token runs
    and the 256-token blocks of the weight-gradient partials) for widths 1..8, both io dtypes, with and without SiLU and bias;
  * the full packed row (32768 tokens, 8 documents, 3*32*128 channels, W=4,
    bf16) on 512 sampled channels;
  * no tokens: the weight and bias gradients are written as zeros;
  * run-to-run identical results (fixed-order reduction of the partials).
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


# 302 tokens: runs of 64 tokens, a second 256-token block with a partial run
# and two empty ones
LENS = [37, 0, 3, 70, 5, 96, 1, 90]
PROMPTS = [12, 0, 0, 20, 4, 32, 0, 40]


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _run(g, dev, cu, prompts, B, x, xn, w, dy, dyn, bias=None, act=0, bf16=False, want_dbias=True):
    import torch
    vl = g.Varlen(cu, prompts, dev)
    out = g.shortconv_dual_bwd(vl, B, to_dev(x, dev, bf16), to_dev(xn, dev, bf16), to_dev(w, dev),
                               to_dev(dy, dev, bf16), to_dev(dyn, dev, bf16),
                               bias=None if bias is None else to_dev(bias, dev), activation=act,
                               want_dbias=want_dbias)
    torch.cuda.synchronize()
    return [None if o is None else to_np(o) for o in out]


@pytest.mark.parametrize("W,bf16", [(1, False), (2, True), (4, False), (4, True), (5, False), (8, True)])
def test_conv_bwd_exact_integers(g, dev, W, bf16):
    """|dx| <= 8 taps * 3 * 8 = 192 < 256: exact in bf16 as well; the weight
    sums stay below 2^24."""
    rng = np.random.default_rng(70 + W)
    cu, B, C = _cu(LENS), 4, 8
    T = int(cu[-1])
    x = rng.integers(-4, 5, (T, C)).astype(np.float32)
    xn = rng.integers(-4, 5, (T, C)).astype(np.float32)
    dy = rng.integers(-4, 5, (T, C)).astype(np.float32)
    dyn = rng.integers(-4, 5, (T, C)).astype(np.float32)
    w = rng.integers(-3, 4, (C, W)).astype(np.float32)
    dx, dxn, dw, db = _run(g, dev, cu, PROMPTS, B, x, xn, w, dy, dyn, bf16=bf16)
    rx, rxn, rw, rb = oracle.shortconv_dual_bwd(cu, PROMPTS, B, x, xn, w, dy, dyn)
    np.testing.assert_array_equal(dx, rx)
    np.testing.assert_array_equal(dxn, rxn)
    np.testing.assert_array_equal(dw, rw)
    np.testing.assert_array_equal(db, rb)


@pytest.mark.parametrize("W,act,bias,bf16", [(1, 0, False, False), (3, 1, True, False), (4, 1, True, True),
                                             (4, 0, False, True), (6, 1, False, True), (7, 0, True, False),
                                             (8, 1, True, True), (2, 1, True, True)])
def test_conv_bwd_ragged(g, dev, W, act, bias, bf16):
    rng = np.random.default_rng(90 + W + 10 * act)
    cu, B, C = _cu(LENS), 4, 48
    T = int(cu[-1])
    rnd = wl.round_bf16 if bf16 else (lambda a: a)
    x = rnd(rng.standard_normal((T, C)).astype(np.float32))
    xn = rnd(rng.standard_normal((T, C)).astype(np.float32))
    dy = rnd(rng.standard_normal((T, C)).astype(np.float32))
    dyn = rnd(rng.standard_normal((T, C)).astype(np.float32))
    w = rng.uniform(-0.5, 0.5, (C, W)).astype(np.float32)
    bb = rng.standard_normal(C).astype(np.float32) if bias else None
    dx, dxn, dw, db = _run(g, dev, cu, PROMPTS, B, x, xn, w, dy, dyn, bias=bb, act=act, bf16=bf16)
    rx, rxn, rw, rb = oracle.shortconv_dual_bwd(cu, PROMPTS, B, x, xn, w, dy, dyn, bias=bb, activation=act)
    tol = TOL_BF16 if bf16 else TOL_F32
    assert rel_rms(dx, rx) <= tol
    assert rel_rms(dxn, rxn) <= tol
    # the weight and bias gradients are fp32 sums in any io dtype
    assert rel_rms(dw, rw) <= TOL_F32
    assert rel_rms(db, rb) <= TOL_F32
    for i, p in enumerate(PROMPTS):
        assert not np.any(dxn[cu[i]:cu[i] + p])


def test_conv_bwd_full_size_sampled_channels(g, dev):
    """One packed row of 32768 tokens, 8 Dirichlet-split docs, 3*32*128 channels,
    W=4, bf16; the oracle checks 512 sampled channels."""
    p = wl.packed_conv()
    T, C = p["x"].shape
    rng = np.random.default_rng(77)
    dy = wl.round_bf16(rng.standard_normal((T, C), dtype=np.float32))
    dyn = wl.round_bf16(rng.standard_normal((T, C), dtype=np.float32))
    dx, dxn, dw, db = _run(g, dev, p["cu_seqlens"], p["prompt_lens"], p["block_size"], p["x"], p["xn"],
                           p["weight"], dy, dyn, bf16=True)
    ch = np.r_[0:256, C - 256:C]
    rx, rxn, rw, rb = oracle.shortconv_dual_bwd(p["cu_seqlens"], p["prompt_lens"], p["block_size"],
                                                np.ascontiguousarray(p["x"][:, ch]),
                                                np.ascontiguousarray(p["xn"][:, ch]),
                                                np.ascontiguousarray(p["weight"][ch]),
                                                np.ascontiguousarray(dy[:, ch]), np.ascontiguousarray(dyn[:, ch]))
    assert rel_rms(dx[:, ch], rx) <= TOL_BF16
    assert rel_rms(dxn[:, ch], rxn) <= TOL_BF16
    assert rel_rms(dw[ch], rw) <= TOL_F32
    assert rel_rms(db[ch], rb) <= TOL_F32


def test_conv_bwd_no_tokens_writes_zero_sums(g, dev):
    import torch
    vl = g.Varlen(np.array([0, 0, 0], np.int32), np.array([0, 0], np.int32), dev)
    C, W = 16, 4
    e = torch.empty((0, C), dtype=torch.bfloat16, device=dev)
    w = torch.ones((C, W), dtype=torch.float32, device=dev)
    dw = torch.full((C, W), float("nan"), device=dev)
    db = torch.full((C,), float("nan"), device=dev)
    g.shortconv_dual_bwd(vl, 4, e, e, w, e, e, out=(torch.empty_like(e), torch.empty_like(e), dw, db))
    torch.cuda.synchronize()
    assert not to_np(dw).any() and not to_np(db).any()


def test_conv_bwd_deterministic_and_optional_bias(g, dev):
    rng = np.random.default_rng(5)
    cu, B, C, W = _cu([300, 211]), 4, 64, 4
    T = int(cu[-1])
    prompts = [100, 48]
    args = [wl.round_bf16(rng.standard_normal((T, C)).astype(np.float32)) for _ in range(2)]
    w = rng.uniform(-0.5, 0.5, (C, W)).astype(np.float32)
    grads = [wl.round_bf16(rng.standard_normal((T, C)).astype(np.float32)) for _ in range(2)]
    a = _run(g, dev, cu, prompts, B, *args, w, *grads, act=1, bf16=True)
    b = _run(g, dev, cu, prompts, B, *args, w, *grads, act=1, bf16=True, want_dbias=False)
    for u, v in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(u, v)
    assert b[3] is None
