"""Strided checkpoints and chunk windows on the chunked bf16 d = 128 path,
through the C ABI.

"FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes, Key
designs item 2): the clean stream keeps only every s-th chunk-start state and
the rest are rebuilt when they are needed.  Here the backward rebuilds them
from the strided checkpoints, as parallel runs of s chunks, and both passes
can run in windows of chunks (per-chunk buffers of one window only, the chain
carried between windows).  The rebuild and the windows repeat the same
arithmetic in the same order, so every output must equal the one-pass,
stride-1 result bit for bit; the one-pass result itself is checked against
the oracle elsewhere, and here once more on integer tags (bit-exact) and on
normal inputs (tolerance)."""
import numpy as np
import pytest

import oracle
from gated_deltanet_dual_amd import workloads as wl
from gpu_util import TOL_BF16, fwd_args, rel_rms, to_dev, to_np
from test_gpu_exact_chunked import bf16_exact, tag_inputs

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dalpha", "dbeta", "dqn", "dkn", "dvn", "dalpha_n", "dbeta_n", "dh0")
IO_GRADS = ("dq", "dk", "dv", "dqn", "dkn", "dvn")
# documents crossing chunk boundaries, empty and sub-chunk ones, prompts at 0,
# at a chunk start and mid-chunk; 13 chunks in the longest
DOCS_LENS = [400, 45, 0, 97, 31, 256, 5, 130]
DOCS_PROMPTS = [12, 0, 0, 64, 28, 96, 4, 100]


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


def inputs(B, seed, flags=0, H=2):
    prompts = [min(n, (p // B) * B) for n, p in zip(DOCS_LENS, DOCS_PROMPTS)]
    inp = wl.gdn_inputs(DOCS_LENS, prompts, H, 128, 128, B, seed=seed, with_h0=True, with_grads=True,
                        normalize_qk=not flags)
    inp.extra["dhf"] = np.random.default_rng(seed + 1).standard_normal((len(DOCS_LENS), H, 128, 128)).astype(
        np.float32)
    return inp


def fwd(g, vl, args, B, h0, flags=0, stride=1, window=0, scale=0.0):
    return g.gdn_dual_fwd(vl, *args, B, h0=h0, flags=flags, scale=scale, want_ckpt=True, ckpt_stride=stride,
                          window=window)


def bwd(g, vl, args, B, ck, do, don, h0, dhf, flags=0, stride=1, window=0, scale=0.0, fws=None):
    return g.gdn_dual_bwd(vl, *args, B, ck, do, don, h0=h0, dh_final=dhf, flags=flags, scale=scale,
                          ckpt_stride=stride, window=window, fwd_workspace=fws)


def ckpt_rows(cu, stride):
    """(document, chunk, slot) of every checkpoint of the given stride."""
    rows = []
    for i in range(len(cu) - 1):
        n = cu[i + 1] - cu[i]
        for c in range(0, (n + 31) // 32, stride):
            rows.append((i, c, cu[i] // (32 * stride) + i + c // stride))
    return rows


@pytest.mark.parametrize("flags", [0, 1])
@pytest.mark.parametrize("stride", [2, 4])
def test_forward_strided_checkpoints(g, dev, stride, flags):
    """Stride-s checkpoints are the stride-1 checkpoints of chunks c % s == 0,
    bit for bit; outputs and final states do not change."""
    import torch
    inp = inputs(4, 700 + stride, flags)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev)
    o1, on1, hf1, ck1 = fwd(g, vl, args, 4, h0, flags)
    o, on, hf, ck = fwd(g, vl, args, 4, h0, flags, stride=stride)
    torch.cuda.synchronize()
    assert ck.shape[0] == g.ckpt_slots(vl, 2, 128, 4, g.BF16, stride)
    for i, c, s in ckpt_rows(inp.cu_seqlens, stride):
        assert torch.equal(ck[s], ck1[inp.cu_seqlens[i] // 32 + i + c]), (i, c)
    assert torch.equal(o, o1) and torch.equal(on, on1) and torch.equal(hf, hf1)


@pytest.mark.parametrize("window", [1, 3, 4, 8, 13])
def test_forward_windows_equal_one_pass(g, dev, window):
    """Windows of 1 .. 13 chunks (13: the longest document in one window,
    with the windowed layout) give the one-pass outputs, final states and
    checkpoints (stride 1 and 2) bit for bit."""
    import torch
    inp = inputs(4, 720 + window)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev)
    ref = fwd(g, vl, args, 4, h0)
    ref2 = fwd(g, vl, args, 4, h0, stride=2)
    got = fwd(g, vl, args, 4, h0, window=window)
    got2 = fwd(g, vl, args, 4, h0, stride=2, window=window)
    torch.cuda.synchronize()
    for x, r in ((got, ref), (got2, ref2)):
        for a, b in zip(x[:3], r[:3]):
            assert torch.equal(a, b)
    # checkpoint slots no chunk maps to (the slot numbering leaves gaps) are never written
    for stride, ck, rk in ((1, got[3], ref[3]), (2, got2[3], ref2[3])):
        for i, c, s in ckpt_rows(inp.cu_seqlens, stride):
            assert torch.equal(ck[s], rk[s]), (stride, i, c)


def test_forward_window_workspace_is_smaller(g, dev):
    inp = inputs(4, 730)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    one = g.workspace_bytes(vl, 2, 128, 4, g.BF16)
    w4 = g.workspace_bytes(vl, 2, 128, 4, g.BF16, window=4)
    assert 0 < w4 < one


@pytest.mark.parametrize("stride,window", [(2, 0), (4, 0), (3, 0), (1, 4), (2, 2), (2, 6), (4, 4), (4, 8), (3, 9)])
def test_backward_stride_and_windows_equal_one_pass(g, dev, stride, window):
    """The reverse mode from stride-s checkpoints (the chunk-start states
    rebuilt in parallel runs), in one pass or in windows, equals the one-pass
    stride-1 reverse mode bit for bit, with h0 and dh_final."""
    import torch
    B = 4
    inp = inputs(B, 740 + 10 * stride + window)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev)
    dhf = to_dev(inp.extra["dhf"], dev)
    do, don = to_dev(inp.do, dev, True), to_dev(inp.don, dev, True)
    _, _, _, ck1 = fwd(g, vl, args, B, h0)
    ref = bwd(g, vl, args, B, ck1, do, don, h0, dhf)
    _, _, _, ck = fwd(g, vl, args, B, h0, stride=stride, window=window)
    got = bwd(g, vl, args, B, ck, do, don, h0, dhf, stride=stride, window=window)
    torch.cuda.synchronize()
    for name in GRADS:
        assert torch.equal(got[name], ref[name]), name


@pytest.mark.parametrize("stride,window", [(2, 4), (4, 0)])
def test_backward_l2_flag_stride_windows(g, dev, stride, window):
    """The q/k L2 flag through the rebuild and the windows: bit for bit the
    one-pass stride-1 reverse mode."""
    import torch
    B = 8
    inp = inputs(B, 760 + stride, flags=1)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev)
    dhf = to_dev(inp.extra["dhf"], dev)
    do, don = to_dev(inp.do, dev, True), to_dev(inp.don, dev, True)
    _, _, _, ck1 = fwd(g, vl, args, B, h0, flags=1)
    ref = bwd(g, vl, args, B, ck1, do, don, h0, dhf, flags=1)
    _, _, _, ck = fwd(g, vl, args, B, h0, flags=1, stride=stride, window=window)
    got = bwd(g, vl, args, B, ck, do, don, h0, dhf, flags=1, stride=stride, window=window)
    torch.cuda.synchronize()
    for name in GRADS:
        assert torch.equal(got[name], ref[name]), name


def test_backward_stride_against_oracle(g, dev):
    """Stride 4 in windows of 4 chunks against the oracle's reverse mode."""
    import torch
    B = 4
    inp = inputs(B, 780)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev)
    dhf = inp.extra["dhf"]
    _, _, _, ck = fwd(g, vl, args, B, h0, stride=4, window=4)
    got = bwd(g, vl, args, B, ck, to_dev(inp.do, dev, True), to_dev(inp.don, dev, True), h0, to_dev(dhf, dev),
              stride=4, window=4)
    torch.cuda.synchronize()
    want = oracle.gdn_dual_bwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), B,
                               inp.do, inp.don, h0=inp.h0, dh_final=dhf)
    for name in GRADS:
        e = rel_rms(to_np(got[name]), want[name])
        assert e <= TOL_BF16, (name, e)


@pytest.mark.parametrize("B", [1, 4, 32])
def test_tags_bit_exact_stride_and_windows(g, dev, B):
    """Integer tags (exact in every precision on the path) through stride-2
    checkpoints and windows of 2 chunks: forward and reverse mode equal the
    oracle bit for bit."""
    import torch
    inp = tag_inputs(B, seed=800 + B, with_grads=True)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev)
    dhf = inp.extra["dhf"]
    o, on, hf, ck = fwd(g, vl, args, B, h0, stride=2, window=2, scale=1.0)
    gr = bwd(g, vl, args, B, ck, to_dev(inp.do, dev, True), to_dev(inp.don, dev, True), h0, to_dev(dhf, dev),
             stride=2, window=2, scale=1.0)
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


def test_full_size_stride4_windows(g, dev):
    """The training-step shape (4 x 8192 tokens, prompt 2048, B = 4, 16
    heads): stride-4 checkpoints and windows of 32 chunks give the one-pass
    stride-1 gradients bit for bit, with a fraction of the workspace."""
    import torch
    B, H = 4, 16
    inp = wl.gdn_inputs([8192] * 4, [2048] * 4, H, 128, 128, B, seed=820, with_grads=True)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    do, don = to_dev(inp.do, dev, True), to_dev(inp.don, dev, True)
    _, _, _, ck1 = fwd(g, vl, args, B, None)
    ref = bwd(g, vl, args, B, ck1, do, don, None, None)
    del ck1
    o, on, _, ck = fwd(g, vl, args, B, None, stride=4, window=32)
    got = bwd(g, vl, args, B, ck, do, don, None, None, stride=4, window=32)
    torch.cuda.synchronize()
    for name in GRADS:
        assert torch.equal(got[name], ref[name]), name
    one = g.workspace_bytes(vl, H, 128, B, g.BF16, for_bwd=True)
    win = g.workspace_bytes(vl, H, 128, B, g.BF16, for_bwd=True, stride=4, window=32)
    assert win * 5 < one, (win, one)
