"""GPU parity of flare_gdn_dual_fwd_route1 (the chunk-then-refine route: every
block-boundary clean state materialised, every noisy block refined from it)
through the C-ABI binding, against the fp64 oracle's dual forward:
  * fp32 io at d = 16 and bf16 io at d = 128, blocks of 4, 16 and 32, ragged
    documents whose last block is partial, an empty document, a document with
    no response, prompts that do and do not start a chunk, initial states;
  * the clean outputs, the noisy outputs (noisy prompt rows exactly 0), the
    final states and the chunk-start states agree with the masked route
    (flare_gdn_dual_fwd) as well as with the oracle;
  * the full dual workload (4 documents x 4096 tokens, prompt 1024, 16 heads,
    d = 128, bf16) at blocks of 4 and 32, the oracle checking two heads.
"""
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


def ref(inp):
    return oracle.gdn_dual_fwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(),
                               inp.block_size, h0=inp.h0)


def run_both(g, inp, dev):
    import torch
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    h0 = to_dev(inp.h0, dev) if inp.h0 is not None else None
    args = fwd_args(inp, dev)
    r1 = g.gdn_dual_fwd_route1(vl, *args, inp.block_size, h0=h0)
    r2 = g.gdn_dual_fwd(vl, *args, inp.block_size, h0=h0, want_ckpt=True)
    torch.cuda.synchronize()
    return r1, r2


def used_ckpt(inp, ck):
    """The chunk-start states that hold a chunk (slot cu_i / 32 + i + c for
    chunk c of document i); the other slots are never written."""
    H = inp.q.shape[1]
    dk, dv = inp.q.shape[2], inp.v.shape[2]
    ck = to_np(ck).reshape(-1, H, dk, dv)
    cu = inp.cu_seqlens
    idx = [cu[i] // 32 + i + c for i in range(len(cu) - 1) for c in range((cu[i + 1] - cu[i] + 31) // 32)]
    return ck[idx]


def check(inp, r1, want, tol, name):
    o, on, hf = to_np(r1[0]), to_np(r1[1]), to_np(r1[2])
    ro, ron, rhf = want
    e = {"o": rel_rms(o, ro), "on": rel_rms(on, ron), "h_final": rel_rms(hf, rhf)}
    print(name, e)
    for key, val in e.items():
        assert val <= tol, (name, key, val)
    for i in range(len(inp.prompt_lens)):
        a, p = inp.cu_seqlens[i], inp.prompt_lens[i]
        assert not np.any(on[a:a + p]), "noisy prompt rows must be written as 0"


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32])
def test_route1_fp32_ragged(g, dev, B):
    # prompts are multiples of B; 48 does not start a chunk at B = 16
    P = [B, 0, 2 * B, 0, 3 * B]
    lens = [P[0] + 5 * B - 1, 0, P[2] + 1, 3, P[4]]  # partial last blocks, an empty doc, no response
    inp = wl.gdn_inputs(lens, P, 3, 16, 16, B, seed=70 + B, io="f32", gates="uniform", with_h0=True)
    r1, r2 = run_both(g, inp, dev)
    check(inp, r1, ref(inp), TOL_F32, "route1_f32_B%d" % B)
    for a, b, name in ((r1[0], r2[0], "o"), (r1[1], r2[1], "on"), (r1[2], r2[2], "h_final")):
        assert rel_rms(to_np(a), to_np(b)) <= TOL_F32, name
    assert rel_rms(used_ckpt(inp, r1[3]), used_ckpt(inp, r2[3])) <= TOL_F32


@pytest.mark.parametrize("B", [4, 16, 32])
def test_route1_bf16_d128(g, dev, B):
    lens, P = [320 + B - 3, 97, 160, 64], [128, 32, 0, 64]
    inp = wl.gdn_inputs(lens, P, 2, 128, 128, B, seed=80 + B, with_h0=True)
    r1, r2 = run_both(g, inp, dev)
    check(inp, r1, ref(inp), TOL_BF16, "route1_bf16_B%d" % B)
    assert rel_rms(to_np(r1[1]), to_np(r2[1])) <= TOL_BF16
    assert rel_rms(used_ckpt(inp, r1[3]), used_ckpt(inp, r2[3])) <= TOL_F32


@pytest.mark.parametrize("B", [4, 32])
def test_route1_dual_full_size(g, dev, B):
    inp = wl.dual_bf16(block_size=B)
    r1, _ = run_both(g, inp, dev)
    check(inp, r1[:3], ref(inp), TOL_BF16, "route1_dual_B%d" % B)
