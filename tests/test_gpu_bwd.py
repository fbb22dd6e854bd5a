"""GPU parity of flare_gdn_dual_bwd (fed by flare_gdn_dual_fwd's checkpoints)
against the oracle's token-level reverse mode, through the C ABI."""
import numpy as np
import pytest

import oracle
from gated_deltanet_dual_amd import workloads as wl
from gpu_util import TOL_BF16, TOL_F32, fwd_args, rel_rms, to_dev, to_np

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


def run_bwd(g, inp, dev, dhf=None, scale=0.0, flags=0):
    import torch
    bf = inp.io == "bf16"
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev) if inp.h0 is not None else None
    _, _, _, ck = g.gdn_dual_fwd(vl, *args, inp.block_size, h0=h0, scale=scale, flags=flags, want_ckpt=True)
    gr = g.gdn_dual_bwd(vl, *args, inp.block_size, ck, to_dev(inp.do, dev, bf), to_dev(inp.don, dev, bf),
                        h0=h0, dh_final=to_dev(dhf, dev) if dhf is not None else None, scale=scale, flags=flags)
    torch.cuda.synchronize()
    return gr


def ref_bwd(inp, dhf=None, scale=0.0, flags=0):
    return oracle.gdn_dual_bwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(),
                               inp.block_size, inp.do, inp.don, h0=inp.h0, dh_final=dhf, scale=scale, flags=flags)


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


def test_bwd_headline_full_size_all_heads(g, dev):
    """4 docs x 8192 tokens (prompt 2048), B=4, H=16, d=128, bf16; the oracle
    checks every head at full length."""
    inp = wl.headline(with_grads=True)
    check(inp, run_bwd(g, inp, dev), ref_bwd(inp), TOL_BF16, "bwd_headline")


def test_bench_step_configuration_full_size(g, dev):
    """The training step exactly as the benchmark times it: the forward into
    caller buffers with the chunk-start states saved, no final state and the
    forward's workspace kept; the backward reading that workspace's chunk
    matrices.  Outputs and all eleven gradients against the oracle, every head
    of the 4 x 8192 workload."""
    import torch
    inp = wl.headline(with_grads=True)
    T, H, d, B = inp.T, inp.H, 128, inp.block_size
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    o = torch.empty((T, H, d), dtype=torch.bfloat16, device=dev)
    on = torch.empty_like(o)
    ckpt = torch.empty((g.ckpt_slots(vl, H, d, B, g.BF16), H, d, d), dtype=torch.float32, device=dev)
    fws = torch.empty((g.workspace_bytes(vl, H, d, B, g.BF16),), dtype=torch.uint8, device=dev)
    ws = torch.empty((g.workspace_bytes(vl, H, d, B, g.BF16, for_bwd=True),), dtype=torch.uint8, device=dev)
    _, _, hf, _ = g.gdn_dual_fwd(vl, *args, B, out=(o, on), ckpt=ckpt, want_h_final=False, workspace=fws)
    assert hf is None
    gr = g.gdn_dual_bwd(vl, *args, B, ckpt, to_dev(inp.do, dev, True), to_dev(inp.don, dev, True),
                        workspace=ws, fwd_workspace=fws)
    torch.cuda.synchronize()
    ro, ron, _ = oracle.gdn_dual_fwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), B)
    e = {"o": rel_rms(to_np(o), ro), "on": rel_rms(to_np(on), ron)}
    print("bench_step fwd", e)
    assert max(e.values()) <= TOL_BF16, e
    check(inp, gr, ref_bwd(inp), TOL_BF16, "bench_step")


def test_bwd_packed_full_size_all_heads(g, dev):
    """One packed row of 32768 tokens, 8 Dirichlet-length documents, 32 heads,
    d=128, bf16 (q/k pre-normalised); the oracle checks every head."""
    lens, prompts = wl.packed_doc_lengths(32768, 8, 4, seed=3)
    inp = wl.gdn_inputs(lens, prompts, 32, 128, 128, 4, seed=13, with_grads=True)
    check(inp, run_bwd(g, inp, dev), ref_bwd(inp), TOL_BF16, "bwd_packed")


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


@pytest.mark.parametrize("B", [4, 1, 32])
def test_bwd_bf16_l2norm_flag(g, dev, B):
    """Reverse mode with the q/k L2 flag on the chunked d = 128 path: the
    gradients w.r.t. the unnormalised q, k of both streams (through the
    normalisation), with h0, dh_final and rows of very different norms."""
    lens = [160, 77, 0, 64, 33]
    prompts = [min(n, (p // B) * B) for n, p in zip(lens, [64, 32, 0, 0, 32])]
    inp = wl.gdn_inputs(lens, prompts, 2, 128, 128, B, seed=90 + B, normalize_qk=False, with_h0=True,
                        with_grads=True)
    rng = np.random.default_rng(91 + B)
    for name in ("q", "k", "qn", "kn"):
        x = getattr(inp, name)
        setattr(inp, name, wl.round_bf16(x * rng.uniform(0.05, 20.0, x.shape[:2] + (1,)).astype(np.float32)))
    dhf = (rng.standard_normal((len(lens), 2, 128, 128)) / 16).astype(np.float32)
    check(inp, run_bwd(g, inp, dev, dhf=dhf, flags=1), ref_bwd(inp, dhf=dhf, flags=oracle.FLAG_QK_L2NORM), TOL_BF16,
          "bwd_l2_B%d" % B)


def test_bwd_l2norm_packed_full_size_all_heads(g, dev):
    """One packed row of 32768 tokens, 8 Dirichlet-length documents, 32 heads,
    d = 128, bf16, q/k normalised by the L2 flag in the forward and the
    reverse mode; every head against the oracle."""
    lens, prompts = wl.packed_doc_lengths(32768, 8, 4, seed=3)
    inp = wl.gdn_inputs(lens, prompts, 32, 128, 128, 4, seed=14, normalize_qk=False, with_grads=True)
    check(inp, run_bwd(g, inp, dev, flags=1), ref_bwd(inp, flags=oracle.FLAG_QK_L2NORM), TOL_BF16, "bwd_l2_packed")


def test_bwd_l2norm_reusing_forward_chunk_matrices(g, dev):
    """With the L2 flag, the backward reading the forward's chunk matrices
    gives the same bits as forming them again."""
    import torch
    inp = wl.gdn_inputs([130, 64, 96], [32, 0, 48], 2, 128, 128, 4, seed=75, normalize_qk=False, with_grads=True)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    fws = torch.empty((g.workspace_bytes(vl, 2, 128, 4, g.BF16, flags=1),), dtype=torch.uint8, device=dev)
    _, _, _, ck = g.gdn_dual_fwd(vl, *args, 4, flags=1, want_ckpt=True, workspace=fws)
    do, don = to_dev(inp.do, dev, True), to_dev(inp.don, dev, True)
    g1 = g.gdn_dual_bwd(vl, *args, 4, ck, do, don, flags=1)
    g2 = g.gdn_dual_bwd(vl, *args, 4, ck, do, don, flags=1, fwd_workspace=fws)
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.equal(g1[k], g2[k]), k


def test_long_document_parallel_runs_full_size(g, dev):
    """One packed row of 32768 tokens holding a single document (prompt 8192),
    16 heads, d = 128, bf16: the state scans run as parallel runs joined by
    their transfer maps; forward and reverse mode against the oracle on every
    head, with h0 and dh_final; the reverse mode also composing with the
    forward's transfer maps (transposed) from the forward's workspace."""
    import torch
    inp = wl.gdn_inputs([32768], [8192], 16, 128, 128, 4, seed=17, with_h0=True, with_grads=True)
    dhf = (np.random.default_rng(18).standard_normal((1, 16, 128, 128)) / 16).astype(np.float32)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev)
    fws = torch.empty((g.workspace_bytes(vl, 16, 128, 4, g.BF16),), dtype=torch.uint8, device=dev)
    o, on, hf, ck = g.gdn_dual_fwd(vl, *args, 4, h0=h0, want_ckpt=True, workspace=fws)
    gr = g.gdn_dual_bwd(vl, *args, 4, ck, to_dev(inp.do, dev, True), to_dev(inp.don, dev, True), h0=h0,
                        dh_final=to_dev(dhf, dev))
    grf = g.gdn_dual_bwd(vl, *args, 4, ck, to_dev(inp.do, dev, True), to_dev(inp.don, dev, True), h0=h0,
                         dh_final=to_dev(dhf, dev), fwd_workspace=fws)
    torch.cuda.synchronize()
    ro, ron, rhf = oracle.gdn_dual_fwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), 4,
                                       h0=inp.h0)
    e = {"o": rel_rms(to_np(o), ro), "on": rel_rms(to_np(on), ron), "h_final": rel_rms(to_np(hf), rhf)}
    print("long_doc fwd", e)
    assert max(e.values()) <= TOL_BF16, e
    want = ref_bwd(inp, dhf=dhf)
    check(inp, gr, want, TOL_BF16, "long_doc")
    check(inp, grf, want, TOL_BF16, "long_doc_fwd_maps")


def test_parallel_runs_long_memory(g, dev):
    """Parallel runs whose transfer maps are far from zero: decays in
    [0.999, 1) per token, so a 2048-token run keeps about e^-1 of its start
    value (with the smooth gates of the other tests the maps underflow to
    zero and the runs' composition reduces to the offsets).  Two documents of
    8192 and 3000 tokens at 16 heads (runs of 64 chunks), h0 and dh_final:
    forward and reverse mode against the oracle, the reverse mode once with
    its own transfer maps and once composing with the forward's (transposed)."""
    import torch
    inp = wl.gdn_inputs([8192, 3000], [100, 36], 16, 128, 128, 4, seed=23, with_h0=True,
                        with_grads=True)
    rng = np.random.default_rng(24)
    inp.alpha = (0.999 + 0.001 * rng.random(inp.alpha.shape)).astype(np.float32)
    inp.alpha_n = (0.999 + 0.001 * rng.random(inp.alpha_n.shape)).astype(np.float32)
    dhf = (rng.standard_normal((2, 16, 128, 128)) / 16).astype(np.float32)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev)
    fws = torch.empty((g.workspace_bytes(vl, 16, 128, 4, g.BF16),), dtype=torch.uint8, device=dev)
    o, on, hf, ck = g.gdn_dual_fwd(vl, *args, 4, h0=h0, want_ckpt=True, workspace=fws)
    do, don = to_dev(inp.do, dev, True), to_dev(inp.don, dev, True)
    gr = g.gdn_dual_bwd(vl, *args, 4, ck, do, don, h0=h0, dh_final=to_dev(dhf, dev))
    grf = g.gdn_dual_bwd(vl, *args, 4, ck, do, don, h0=h0, dh_final=to_dev(dhf, dev), fwd_workspace=fws)
    torch.cuda.synchronize()
    ro, ron, rhf = oracle.gdn_dual_fwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), 4,
                                       h0=inp.h0)
    e = {"o": rel_rms(to_np(o), ro), "on": rel_rms(to_np(on), ron), "h_final": rel_rms(to_np(hf), rhf)}
    print("long_memory fwd", e)
    assert max(e.values()) <= TOL_BF16, e
    want = ref_bwd(inp, dhf=dhf)
    check(inp, gr, want, TOL_BF16, "long_memory")
    check(inp, grf, want, TOL_BF16, "long_memory_fwd_maps")


def test_parallel_runs_ragged_documents(g, dev):
    """Two documents of 8192 and 3010 tokens (prompts 256, 64) at 16 heads:
    runs of 64 chunks, the shorter document with a partial last run; every
    checkpoint is the clean state after 32c tokens of its document."""
    import torch
    inp = wl.gdn_inputs([8192, 3010], [256, 64], 16, 128, 128, 2, seed=19, with_h0=True, with_grads=True)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev)
    o, on, hf, ck = g.gdn_dual_fwd(vl, *args, 2, h0=h0, want_ckpt=True)
    gr = g.gdn_dual_bwd(vl, *args, 2, ck, to_dev(inp.do, dev, True), to_dev(inp.don, dev, True), h0=h0)
    torch.cuda.synchronize()
    ro, ron, rhf = oracle.gdn_dual_fwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), 2,
                                       h0=inp.h0)
    e = {"o": rel_rms(to_np(o), ro), "on": rel_rms(to_np(on), ron), "h_final": rel_rms(to_np(hf), rhf)}
    assert max(e.values()) <= TOL_BF16, e
    check(inp, gr, ref_bwd(inp), TOL_BF16, "runs_ragged")
    # a few checkpoint slots across run boundaries of the second document
    ck = to_np(ck)
    cu = inp.cu_seqlens
    for c in (0, 63, 64, 65, 94):
        L = 32 * c
        sl = slice(cu[1], cu[1] + L)
        pre = [x[sl] for x in inp.clean_args() + inp.noisy_args()]
        _, _, st = oracle.gdn_dual_fwd([0, L], [L], *pre, 2, h0=inp.h0[1:2])
        assert rel_rms(ck[cu[1] // 32 + 1 + c], st[0]) <= 1e-4, c
