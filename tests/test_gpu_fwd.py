"""GPU parity of flare_gdn_dual_fwd against the fp64 oracle (called through the
C ABI).  Sizes span several chunks and d_v tiles with ragged document tails;
the full-size workloads are checked on every head."""
import numpy as np
import pytest

import oracle
from gated_deltanet_dual_amd import workloads as wl
from gpu_util import TOL_BF16, TOL_F32, fwd_args, rel_rms, to_dev, to_np

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


def run(g, inp, dev, flags=0, scale=0.0, want_ckpt=False):
    import torch
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    h0 = to_dev(inp.h0, dev) if inp.h0 is not None else None
    o, on, hf, ck = g.gdn_dual_fwd(vl, *fwd_args(inp, dev), inp.block_size, h0=h0, flags=flags,
                                   scale=scale, want_ckpt=want_ckpt)
    torch.cuda.synchronize()
    return o, on, hf, ck


def ref(inp, flags=0, scale=0.0):
    return oracle.gdn_dual_fwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(),
                               inp.block_size, h0=inp.h0, flags=flags, scale=scale)


def check(inp, got, want, tol, name=""):
    o, on, hf = to_np(got[0]), to_np(got[1]), to_np(got[2])
    ro, ron, rhf = want
    e = {"o": rel_rms(o, ro), "on": rel_rms(on, ron), "h_final": rel_rms(hf, rhf)}
    print(name, e)
    for key, val in e.items():
        assert val <= tol, (name, key, val)
    # noisy prompt rows are exactly zero
    for i in range(len(inp.prompt_lens)):
        a, p = inp.cu_seqlens[i], inp.prompt_lens[i]
        assert not np.any(on[a:a + p]), "noisy prompt rows must be written as 0"


def test_tiny_fp32(g, dev):
    """1 doc of 64 tokens, prompt 16, B=4, H=1, d=16, fp32."""
    inp = wl.tiny_fp32()
    check(inp, run(g, inp, dev), ref(inp), TOL_F32, "tiny_fp32")


def test_fp32_ragged_docs_and_h0(g, dev):
    inp = wl.gdn_inputs([64, 45, 0, 100, 3], [16, 8, 0, 0, 0], 3, 16, 16, 4, seed=11, io="f32",
                        gates="uniform", with_h0=True)
    check(inp, run(g, inp, dev), ref(inp), TOL_F32, "fp32_ragged")


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32])
def test_bf16_block_sizes(g, dev, B):
    inp = wl.gdn_inputs([320, 97, 160], [128, 32, 0], 2, 128, 128, B, seed=20 + B)
    check(inp, run(g, inp, dev), ref(inp), TOL_BF16, "bf16_B%d" % B)


def test_bf16_h0_scale_and_empty_docs(g, dev):
    inp = wl.gdn_inputs([0, 200, 0, 33, 64], [0, 40, 0, 32, 64], 3, 128, 128, 4, seed=31, with_h0=True)
    check(inp, run(g, inp, dev, scale=0.3), ref(inp, scale=0.3), TOL_BF16, "bf16_h0")


def test_bf16_l2norm_flag(g, dev):
    inp = wl.gdn_inputs([150, 90], [48, 0], 2, 128, 128, 4, seed=32, normalize_qk=False)
    check(inp, run(g, inp, dev, flags=1), ref(inp, flags=oracle.FLAG_QK_L2NORM), TOL_BF16, "bf16_l2")


@pytest.mark.parametrize("B", [1, 8, 32])
def test_bf16_l2norm_flag_chunked_ragged(g, dev, B):
    """The q/k L2 flag on the chunked d = 128 path (folded into per-row
    factors): ragged, empty and sub-chunk documents, prompts mid-chunk, h0,
    unnormalised q/k of varied scale, checkpoints equal to the unflagged
    forward's on normalised inputs where those are exact."""
    lens = [200, 0, 45, 97, 31, 64]
    prompts = [min(n, (p // B) * B) for n, p in zip(lens, [40, 0, 12, 64, 28, 0])]
    inp = wl.gdn_inputs(lens, prompts, 3, 128, 128, B, seed=40 + B, normalize_qk=False, with_h0=True)
    rng = np.random.default_rng(B)
    for name in ("q", "k", "qn", "kn"):  # rows of very different norms
        x = getattr(inp, name)
        setattr(inp, name, wl.round_bf16(x * rng.uniform(0.05, 20.0, x.shape[:2] + (1,)).astype(np.float32)))
    got = run(g, inp, dev, flags=1, want_ckpt=True)
    check(inp, got, ref(inp, flags=oracle.FLAG_QK_L2NORM), TOL_BF16, "bf16_l2_B%d" % B)


def test_d16_bf16(g, dev):
    inp = wl.gdn_inputs([77, 64], [20, 4], 4, 16, 16, 4, seed=33)
    check(inp, run(g, inp, dev), ref(inp), TOL_BF16, "d16_bf16")


def test_checkpoints_are_chunk_start_states(g, dev):
    """ckpt slot floor(cu_i/32)+i+c holds the clean state after 32c tokens of doc i."""
    inp = wl.gdn_inputs([100, 64, 7], [0, 32, 4], 2, 16, 16, 4, seed=34, io="f32", gates="uniform",
                        with_h0=True)
    _, _, _, ck = run(g, inp, dev, want_ckpt=True)
    ck = to_np(ck)
    cu = inp.cu_seqlens
    for i in range(3):
        n = cu[i + 1] - cu[i]
        for c in range((n + 31) // 32):
            L = 32 * c
            sl = slice(cu[i], cu[i] + L)
            pre = [x[sl] for x in inp.clean_args() + inp.noisy_args()]
            _, _, hf = oracle.gdn_dual_fwd([0, L], [L], *pre, 4, h0=inp.h0[i:i + 1])
            slot = cu[i] // 32 + i + c
            assert rel_rms(ck[slot], hf[0]) <= TOL_F32, (i, c)


def test_checkpoints_chunked_path(g, dev):
    """bf16 io at d = 128 (chunk pre-pass + state scan + output pass): every
    checkpoint slot holds the clean state after 32c tokens of its document
    (empty and sub-chunk documents included), and the outputs are the same
    bits whether checkpoints are asked for or not."""
    import torch
    inp = wl.gdn_inputs([100, 0, 64, 7, 45], [0, 0, 32, 4, 44], 2, 128, 128, 4, seed=35, with_h0=True)
    o1, on1, hf1, ck = run(g, inp, dev, want_ckpt=True)
    o2, on2, hf2, _ = run(g, inp, dev)
    assert torch.equal(o1, o2) and torch.equal(on1, on2) and torch.equal(hf1, hf2)
    ck = to_np(ck)
    cu = inp.cu_seqlens
    for i in range(len(inp.prompt_lens)):
        n = cu[i + 1] - cu[i]
        for c in range((n + 31) // 32):
            L = 32 * c
            sl = slice(cu[i], cu[i] + L)
            pre = [x[sl] for x in inp.clean_args() + inp.noisy_args()]
            _, _, hf = oracle.gdn_dual_fwd([0, L], [L], *pre, 4, h0=inp.h0[i:i + 1])
            slot = cu[i] // 32 + i + c
            assert rel_rms(ck[slot], hf[0]) <= TOL_F32, (i, c, rel_rms(ck[slot], hf[0]))


def test_exact_tags_bit_identical(g, dev):
    """fp32, a = b = 1, standard-basis keys and small-integer values: every
    intermediate is an exact small integer, so GPU and oracle agree bit for bit,
    which pins the block, document and chunk-boundary selection."""
    rng = np.random.default_rng(35)
    lens, prompts, H, d, B = [70, 33, 64, 1], [12, 0, 64, 0], 2, 16, 4
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    eye = np.eye(d, dtype=np.float32)

    def keys():
        return eye[rng.integers(0, d, size=(T, H))]

    inp = wl.gdn_inputs(lens, prompts, H, d, d, B, seed=0, io="f32", gates="uniform")
    inp.q, inp.k, inp.qn, inp.kn = keys(), keys(), keys(), keys()
    inp.v = rng.integers(-3, 4, size=(T, H, d)).astype(np.float32)
    inp.vn = rng.integers(-3, 4, size=(T, H, d)).astype(np.float32)
    for name in ("alpha", "beta", "alpha_n", "beta_n"):
        setattr(inp, name, np.ones((T, H), np.float32))
    got = run(g, inp, dev, scale=1.0)
    want = ref(inp, scale=1.0)
    np.testing.assert_array_equal(to_np(got[0]), want[0])
    np.testing.assert_array_equal(to_np(got[1]), want[1])
    np.testing.assert_array_equal(to_np(got[2]), want[2])


def test_invariants_bit_exact(g, dev):
    """Clean outputs do not depend on noisy inputs; packing equals separate
    documents; two runs are bit-identical."""
    import torch
    inp = wl.gdn_inputs([130, 64, 95], [32, 0, 60], 2, 128, 128, 4, seed=36)
    o1, on1, hf1, _ = run(g, inp, dev)
    o2, on2, hf2, _ = run(g, inp, dev)
    assert torch.equal(o1, o2) and torch.equal(on1, on2) and torch.equal(hf1, hf2)
    alt = wl.gdn_inputs([130, 64, 95], [32, 0, 60], 2, 128, 128, 4, seed=99)
    inp2 = wl.gdn_inputs([130, 64, 95], [32, 0, 60], 2, 128, 128, 4, seed=36)
    inp2.qn, inp2.kn, inp2.vn, inp2.alpha_n, inp2.beta_n = alt.qn, alt.kn, alt.vn, alt.alpha_n, alt.beta_n
    o3, _, hf3, _ = run(g, inp2, dev)
    assert torch.equal(o1, o3) and torch.equal(hf1, hf3)
    cu = inp.cu_seqlens
    for i in range(3):
        sl = slice(cu[i], cu[i + 1])
        one = wl.gdn_inputs([cu[i + 1] - cu[i]], [inp.prompt_lens[i]], 2, 128, 128, 4, seed=0)
        for name in ("q", "k", "v", "alpha", "beta", "qn", "kn", "vn", "alpha_n", "beta_n"):
            setattr(one, name, np.ascontiguousarray(getattr(inp, name)[sl]))
        oi, oni, hfi, _ = run(g, one, dev)
        assert torch.equal(oi, o1[sl]) and torch.equal(oni, on1[sl]) and torch.equal(hfi[0], hf1[i])


def test_headline_full_size_all_heads(g, dev):
    """4 docs x 8192 tokens (prompt 2048), B=4, 16 heads, d=128, bf16 -- the
    benchmark's launch; the oracle checks every head at full length."""
    inp = wl.headline(with_grads=False)
    got = run(g, inp, dev)
    check(inp, got, ref(inp), TOL_BF16, "headline")


@pytest.mark.parametrize("B", [4, 8, 16, 32])
def test_dual_bf16_full_size_block_sweep(g, dev, B):
    """4 docs x 4096 tokens (prompt 1024), 16 heads, d=128, bf16, block sizes
    4..32 at full size; the oracle checks every head at full length."""
    inp = wl.dual_bf16(block_size=B)
    check(inp, run(g, inp, dev), ref(inp), TOL_BF16, "dual_bf16_B%d" % B)


def test_packed_l2norm_full_size(g, dev):
    """One packed row of 32768 tokens holding 8 Dirichlet-length documents
    (prompt fraction U[0.1,0.5]), 32 heads, d=128, bf16, q/k normalised by the
    forward's L2 flag; the oracle checks every head."""
    lens, prompts = wl.packed_doc_lengths(32768, 8, 4, seed=3)
    inp = wl.gdn_inputs(lens, prompts, 32, 128, 128, 4, seed=3, normalize_qk=False)
    check(inp, run(g, inp, dev, flags=g.QK_L2NORM), ref(inp, flags=oracle.FLAG_QK_L2NORM), TOL_BF16, "packed_l2")
