"""GPU edge cases through the C-ABI binding, against the fp64 oracle: batches
whose documents are all empty (T = 0).  The forward must still hand each
document's initial state through as its final state, the reverse mode must
hand dh_final through as dh0 (zero without it), and the chunk-then-refine
forward must do the same as the masked one.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_dual_amd import workloads as wl
from gpu_util import fwd_args, rel_rms, to_dev, to_np

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


CASES = [(128, "bf16"), (16, "f32")]


@pytest.mark.parametrize("d,io", CASES)
def test_all_empty_documents_forward(g, dev, d, io):
    import torch
    inp = wl.gdn_inputs([0, 0, 0], [0, 0, 0], 2, d, d, 4, seed=90 + d, io=io, with_h0=True)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    _, _, hf, _ = g.gdn_dual_fwd(vl, *fwd_args(inp, dev), 4, h0=to_dev(inp.h0, dev), want_ckpt=True)
    torch.cuda.synchronize()
    _, _, rhf = oracle.gdn_dual_fwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), 4,
                                    h0=inp.h0)
    assert rel_rms(to_np(hf), rhf) <= 1e-7
    assert rel_rms(to_np(hf), inp.h0) <= 1e-7


@pytest.mark.parametrize("d,io", CASES)
def test_all_empty_documents_backward(g, dev, d, io):
    import torch
    inp = wl.gdn_inputs([0, 0], [0, 0], 2, d, d, 4, seed=92 + d, io=io, with_h0=True, with_grads=True)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    h0 = to_dev(inp.h0, dev)
    _, _, _, ck = g.gdn_dual_fwd(vl, *args, 4, h0=h0, want_ckpt=True)
    bf = io == "bf16"
    dhf = np.random.default_rng(93).standard_normal(inp.h0.shape).astype(np.float32)
    gr = g.gdn_dual_bwd(vl, *args, 4, ck, to_dev(inp.do, dev, bf), to_dev(inp.don, dev, bf), h0=h0,
                        dh_final=to_dev(dhf, dev))
    gr0 = g.gdn_dual_bwd(vl, *args, 4, ck, to_dev(inp.do, dev, bf), to_dev(inp.don, dev, bf), h0=h0)
    torch.cuda.synchronize()
    ref = oracle.gdn_dual_bwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), 4, inp.do,
                              inp.don, h0=inp.h0, dh_final=dhf)
    assert rel_rms(to_np(gr["dh0"]), ref["dh0"]) <= 1e-7
    assert rel_rms(to_np(gr["dh0"]), dhf) <= 1e-7
    assert not to_np(gr0["dh0"]).any()


@pytest.mark.parametrize("d,io", CASES)
def test_all_empty_documents_route1(g, dev, d, io):
    import torch
    inp = wl.gdn_inputs([0, 0, 0], [0, 0, 0], 2, d, d, 4, seed=94 + d, io=io, with_h0=True)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    _, _, hf, _ = g.gdn_dual_fwd_route1(vl, *fwd_args(inp, dev), 4, h0=to_dev(inp.h0, dev))
    torch.cuda.synchronize()
    assert rel_rms(to_np(hf), inp.h0) <= 1e-7
