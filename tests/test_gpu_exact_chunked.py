"""Bit-exact integer-tag parity of the chunked bf16 d = 128 kernels (the
headline path), forward and reverse mode, through the C ABI.

With alpha = beta = 1, standard-basis keys and queries, small-integer values,
initial states, upstream gradients and scale 1, the gated delta rule of "FLARE:
Diffusion for Hybrid Language Model" (papernotes.org notes, Key designs item 2)
only copies and adds small integers: a write replaces the row of S that its key
selects, a read returns one row.  Every value of the chunked form is then an
integer far below 2^16 -- exact in bf16, in the hi/lo bf16 splits of the fp32
operands and in fp32 accumulation, whatever the order -- so the GPU must agree
with the fp64 oracle bit for bit (after the bf16 rounding of the stored
outputs, which both sides round to nearest-even).  Any slip in the block,
document, prompt or chunk-boundary selection moves a row and shows.

Documents cross chunk boundaries, prompts start at 0, at a chunk start and in
the middle of a chunk, and there are empty, sub-chunk and one-chunk documents.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_dual_amd import workloads as wl
from gpu_util import fwd_args, to_dev, to_np

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dalpha", "dbeta", "dqn", "dkn", "dvn", "dalpha_n", "dbeta_n", "dh0")
IO_GRADS = ("dq", "dk", "dv", "dqn", "dkn", "dvn")

# (length, wanted prompt); the prompt is rounded down to a multiple of B
DOCS = [(200, 12), (45, 0), (0, 0), (97, 64), (31, 28), (32, 32), (64, 0), (5, 4), (130, 100), (257, 36)]


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


def tag_inputs(B, seed, H=2, d=128, docs=DOCS, with_grads=False):
    lens = [n for n, _ in docs]
    prompts = [min(n, (p // B) * B) for n, p in docs]
    T = sum(lens)
    rng = np.random.default_rng(seed)
    eye = np.eye(d, dtype=np.float32)
    inp = wl.gdn_inputs(lens, prompts, H, d, d, B, seed=0, io="bf16", gates="uniform")

    def keys():
        return eye[rng.integers(0, d, size=(T, H))]

    def ints(shape, lo=-3, hi=3):
        return rng.integers(lo, hi + 1, size=shape).astype(np.float32)

    inp.q, inp.k, inp.qn, inp.kn = keys(), keys(), keys(), keys()
    inp.v, inp.vn = ints((T, H, d)), ints((T, H, d))
    for name in ("alpha", "beta", "alpha_n", "beta_n"):
        setattr(inp, name, np.ones((T, H), np.float32))
    inp.h0 = ints((len(lens), H, d, d), -2, 2)
    if with_grads:
        inp.do, inp.don = ints((T, H, d), -2, 2), ints((T, H, d), -2, 2)
        inp.extra["dhf"] = ints((len(lens), H, d, d), -2, 2)
    return inp


def bf16_exact(x):
    """The bf16 value the kernels store for an exact fp64 result (nearest-even)."""
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.abs(x) < 2 ** 24) and np.all(x == np.round(x)), "tag values must be small integers"
    return wl.round_bf16(x.astype(np.float32)).astype(np.float64)


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32])
def test_forward_tags_bit_exact(g, dev, B):
    import torch
    inp = tag_inputs(B, seed=100 + B)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    h0 = to_dev(inp.h0, dev)
    o, on, hf, ck = g.gdn_dual_fwd(vl, *fwd_args(inp, dev), B, h0=h0, scale=1.0, want_ckpt=True)
    torch.cuda.synchronize()
    ro, ron, rhf = oracle.gdn_dual_fwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), B,
                                       h0=inp.h0, scale=1.0)
    np.testing.assert_array_equal(to_np(o), bf16_exact(ro))
    np.testing.assert_array_equal(to_np(on), bf16_exact(ron))
    np.testing.assert_array_equal(to_np(hf), rhf)
    # every checkpoint slot: the clean state after 32c tokens of its document
    ck = to_np(ck)
    cu = inp.cu_seqlens
    for i in range(len(inp.prompt_lens)):
        n = cu[i + 1] - cu[i]
        for c in range((n + 31) // 32):
            L = 32 * c
            sl = slice(cu[i], cu[i] + L)
            pre = [x[sl] for x in inp.clean_args() + inp.noisy_args()]
            _, _, st = oracle.gdn_dual_fwd([0, L], [L], *pre, B, h0=inp.h0[i:i + 1], scale=1.0)
            np.testing.assert_array_equal(ck[cu[i] // 32 + i + c], st[0], err_msg="doc %d chunk %d" % (i, c))


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32])
def test_backward_tags_bit_exact(g, dev, B):
    """The reverse mode on the same tags, reading the forward's chunk matrices
    (the training step's configuration) and, separately, forming its own."""
    import torch
    inp = tag_inputs(B, seed=200 + B, with_grads=True)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev)
    dhf = inp.extra["dhf"]
    fws = torch.empty((g.workspace_bytes(vl, inp.H, 128, B, g.BF16),), dtype=torch.uint8, device=dev)
    _, _, _, ck = g.gdn_dual_fwd(vl, *args, B, h0=h0, scale=1.0, want_ckpt=True, want_h_final=False,
                                 workspace=fws)
    do, don = to_dev(inp.do, dev, True), to_dev(inp.don, dev, True)
    g1 = g.gdn_dual_bwd(vl, *args, B, ck, do, don, h0=h0, dh_final=to_dev(dhf, dev), scale=1.0,
                        fwd_workspace=fws)
    g2 = g.gdn_dual_bwd(vl, *args, B, ck, do, don, h0=h0, dh_final=to_dev(dhf, dev), scale=1.0)
    torch.cuda.synchronize()
    want = oracle.gdn_dual_bwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), B,
                               inp.do, inp.don, h0=inp.h0, dh_final=dhf, scale=1.0)
    for name in GRADS:
        ref = bf16_exact(want[name]) if name in IO_GRADS else want[name]
        np.testing.assert_array_equal(to_np(g1[name]), ref, err_msg=name)
        assert torch.equal(g1[name], g2[name]), name


def test_tags_bit_exact_through_parallel_runs(g, dev):
    """A document long enough, with few enough chains, that the state scans
    run as parallel runs joined by their transfer maps (one 8192-token and one
    3000-token document at 16 heads): forward and reverse mode still equal the
    oracle bit for bit on the integer tags (the transfer maps and offsets of
    the runs are then integer matrices too).  The reverse mode runs twice:
    forming its own transfer maps, and composing with the forward's
    (transposed) from the forward's workspace."""
    import torch
    docs = [(8192, 100), (3000, 36)]
    B = 4
    inp = tag_inputs(B, seed=400, H=16, docs=docs, with_grads=True)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev)
    dhf = inp.extra["dhf"]
    fws = torch.empty((g.workspace_bytes(vl, inp.H, 128, B, g.BF16),), dtype=torch.uint8, device=dev)
    o, on, hf, ck = g.gdn_dual_fwd(vl, *args, B, h0=h0, scale=1.0, want_ckpt=True, workspace=fws)
    gr = g.gdn_dual_bwd(vl, *args, B, ck, to_dev(inp.do, dev, True), to_dev(inp.don, dev, True), h0=h0,
                        dh_final=to_dev(dhf, dev), scale=1.0)
    grf = g.gdn_dual_bwd(vl, *args, B, ck, to_dev(inp.do, dev, True), to_dev(inp.don, dev, True), h0=h0,
                         dh_final=to_dev(dhf, dev), scale=1.0, fwd_workspace=fws)
    torch.cuda.synchronize()
    ro, ron, rhf = oracle.gdn_dual_fwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), B,
                                       h0=inp.h0, scale=1.0)
    np.testing.assert_array_equal(to_np(o), bf16_exact(ro))
    np.testing.assert_array_equal(to_np(on), bf16_exact(ron))
    np.testing.assert_array_equal(to_np(hf), rhf)
    want = oracle.gdn_dual_bwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), B,
                               inp.do, inp.don, h0=inp.h0, dh_final=dhf, scale=1.0)
    for name in GRADS:
        ref = bf16_exact(want[name]) if name in IO_GRADS else want[name]
        np.testing.assert_array_equal(to_np(gr[name]), ref, err_msg=name)
        np.testing.assert_array_equal(to_np(grf[name]), ref, err_msg=name + " (forward's maps)")
