"""GPU parity of flare_gdn_dual_bwd (fed by flare_gdn_dual_fwd's checkpoints)
against the oracle's token-level reverse mode, through the C ABI."""
import numpy as np
import pytest

import oracle
from gated_deltanet_dual_amd import workloads as wl
from gpu_util import TOL_BF16, TOL_F32, fwd_args, rel_rms, sub_heads, to_dev, to_np

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dalpha", "dbeta", "dqn", "dkn", "dvn", "dalpha_n", "dbeta_n", "dh0")


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


def run_bwd(g, inp, dev, dhf=None, scale=0.0):
    import torch
    bf = inp.io == "bf16"
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev) if inp.h0 is not None else None
    _, _, _, ck = g.gdn_dual_fwd(vl, *args, inp.block_size, h0=h0, scale=scale, want_ckpt=True)
    gr = g.gdn_dual_bwd(vl, *args, inp.block_size, ck, to_dev(inp.do, dev, bf), to_dev(inp.don, dev, bf),
                        h0=h0, dh_final=to_dev(dhf, dev) if dhf is not None else None, scale=scale)
    torch.cuda.synchronize()
    return gr


def ref_bwd(inp, dhf=None, scale=0.0):
    return oracle.gdn_dual_bwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(),
                               inp.block_size, inp.do, inp.don, h0=inp.h0, dh_final=dhf, scale=scale)


def check(inp, got, want, tol, name):
    errs = {k: rel_rms(to_np(got[k]), want[k]) for k in GRADS}
    print(name, {k: "%.2e" % v for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= tol, (name, k, e)
    for i in range(len(inp.prompt_lens)):
        a, p = inp.cu_seqlens[i], inp.prompt_lens[i]
        for k in ("dqn", "dkn", "dvn", "dalpha_n", "dbeta_n"):
            assert not np.any(to_np(got[k])[a:a + p]), (name, k, "noisy prompt rows must be 0")


def test_bwd_tiny_fp32(g, dev):
    inp = wl.gdn_inputs([64], [16], 1, 16, 16, 4, seed=61, io="f32", gates="uniform", with_grads=True)
    check(inp, run_bwd(g, inp, dev), ref_bwd(inp), TOL_F32, "bwd_tiny_fp32")


def test_bwd_fp32_ragged_h0_dhfinal(g, dev):
    inp = wl.gdn_inputs([70, 33, 0, 96, 5], [16, 0, 0, 40, 4], 2, 16, 16, 4, seed=62, io="f32",
                        gates="uniform", with_h0=True, with_grads=True)
    dhf = np.random.default_rng(63).standard_normal((5, 2, 16, 16)).astype(np.float32)
    check(inp, run_bwd(g, inp, dev, dhf=dhf, scale=0.3), ref_bwd(inp, dhf=dhf, scale=0.3), TOL_F32,
          "bwd_fp32_ragged")


@pytest.mark.parametrize("B", [4, 1, 8, 32])
def test_bwd_bf16(g, dev, B):
    inp = wl.gdn_inputs([160, 77, 64], [64, 32, 0], 2, 128, 128, B, seed=64 + B, with_grads=True)
    check(inp, run_bwd(g, inp, dev), ref_bwd(inp), TOL_BF16, "bwd_bf16_B%d" % B)


def test_bwd_bf16_edge_documents(g, dev):
    """The chunked d = 128 path on the degenerate documents: empty, shorter
    than a chunk, exactly one chunk, all prompt, no prompt, a ragged tail;
    with h0, dh_final and an explicit scale."""
    lens, plens = [0, 5, 31, 32, 0, 64, 97, 40], [0, 4, 28, 32, 0, 0, 64, 40]
    inp = wl.gdn_inputs(lens, plens, 2, 128, 128, 4, seed=73, with_h0=True, with_grads=True)
    dhf = (np.random.default_rng(74).standard_normal((len(lens), 2, 128, 128)) / 16).astype(np.float32)
    check(inp, run_bwd(g, inp, dev, dhf=dhf, scale=0.2), ref_bwd(inp, dhf=dhf, scale=0.2), TOL_BF16,
          "bwd_bf16_edge")


def test_bwd_bf16_h0(g, dev):
    inp = wl.gdn_inputs([100, 37], [20, 0], 2, 128, 128, 4, seed=70, with_h0=True, with_grads=True)
    dhf = (np.random.default_rng(71).standard_normal((2, 2, 128, 128)) / 16).astype(np.float32)
    check(inp, run_bwd(g, inp, dev, dhf=dhf), ref_bwd(inp, dhf=dhf), TOL_BF16, "bwd_bf16_h0")


def test_bwd_deterministic(g, dev):
    import torch
    inp = wl.gdn_inputs([130, 64], [32, 0], 2, 128, 128, 4, seed=72, with_grads=True)
    g1, g2 = run_bwd(g, inp, dev), run_bwd(g, inp, dev)
    for k in GRADS:
        assert torch.equal(g1[k], g2[k]), k


def test_bwd_headline_full_size_sampled_heads(g, dev):
    """4 docs x 8192 tokens (prompt 2048), B=4, H=16, d=128, bf16; the oracle
    checks heads 3 and 12 at full length."""
    inp = wl.headline(with_grads=True)
    gr = run_bwd(g, inp, dev)
    heads = [3, 12]
    sub = sub_heads(inp, heads)
    want = ref_bwd(sub)
    got = {k: (v[:, heads] if k != "dh0" else v[:, heads]) for k, v in gr.items()}
    check(sub, got, want, TOL_BF16, "bwd_headline")


def test_bwd_packed_full_size_sampled_heads(g, dev):
    """One packed row of 32768 tokens, 8 Dirichlet-length documents, 32 heads,
    d=128, bf16 (q/k pre-normalised); the oracle checks heads 7 and 24."""
    lens, prompts = wl.packed_doc_lengths(32768, 8, 4, seed=3)
    inp = wl.gdn_inputs(lens, prompts, 32, 128, 128, 4, seed=13, with_grads=True)
    gr = run_bwd(g, inp, dev)
    heads = [7, 24]
    sub = sub_heads(inp, heads)
    check(sub, {k: v[:, heads] for k, v in gr.items()}, ref_bwd(sub), TOL_BF16, "bwd_packed")


def test_bwd_reusing_forward_chunk_matrices_is_identical(g, dev):
    """Passing the forward's workspace lets the backward read its chunk
    matrices instead of forming them again; the gradients are bit-identical."""
    import torch
    inp = wl.gdn_inputs([130, 64, 96], [32, 0, 48], 2, 128, 128, 4, seed=74, with_grads=True)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    fws = torch.empty((g.workspace_bytes(vl, 2, 128, 4, g.BF16),), dtype=torch.uint8, device=dev)
    _, _, _, ck = g.gdn_dual_fwd(vl, *args, 4, want_ckpt=True, workspace=fws)
    do, don = to_dev(inp.do, dev, True), to_dev(inp.don, dev, True)
    g1 = g.gdn_dual_bwd(vl, *args, 4, ck, do, don)
    g2 = g.gdn_dual_bwd(vl, *args, 4, ck, do, don, fwd_workspace=fws)
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.equal(g1[k], g2[k]), k
