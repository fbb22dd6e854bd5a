"""The torch.autograd wrapper (gated_deltanet_dual_amd.autograd.gdn_dual):
gradients of a loss through o, o~ and h_final equal the library's reverse
mode called directly (bit for bit) and the oracle's (within the bf16
tolerance); without an h0 no gradient is returned for it."""
import numpy as np
import pytest

import oracle
from gated_deltanet_dual_amd import workloads as wl
from gpu_util import TOL_BF16, fwd_args, rel_rms, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


@pytest.mark.parametrize("flags", [0, 1])
def test_autograd_matches_reverse_mode(dev, flags):
    import torch
    import gated_deltanet_dual_amd as g
    from gated_deltanet_dual_amd.autograd import gdn_dual
    inp = wl.gdn_inputs([130, 64, 96], [32, 0, 48], 2, 128, 128, 4, seed=80 + flags, with_h0=True, with_grads=True,
                        normalize_qk=flags == 0)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    leaves = [t.clone().requires_grad_(True) for t in fwd_args(inp, dev)]
    h0 = to_dev(inp.h0, dev).requires_grad_(True)
    o, on, hf = gdn_dual(vl, *leaves, 4, h0=h0, flags=flags)
    do, don = to_dev(inp.do, dev, True), to_dev(inp.don, dev, True)
    dhf = to_dev((np.random.default_rng(5).standard_normal(hf.shape) / 16).astype(np.float32), dev)
    loss = (o.float() * do.float()).sum() + (on.float() * don.float()).sum() + (hf * dhf).sum()
    loss.backward()
    # the reverse mode called directly with the same output gradients
    args = fwd_args(inp, dev)
    _, _, _, ck = g.gdn_dual_fwd(vl, *args, 4, h0=to_dev(inp.h0, dev), flags=flags, want_ckpt=True)
    direct = g.gdn_dual_bwd(vl, *args, 4, ck, do, don, h0=to_dev(inp.h0, dev), dh_final=dhf, flags=flags)
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dalpha", "dbeta", "dqn", "dkn", "dvn", "dalpha_n", "dbeta_n")
    for name, leaf in zip(names, leaves):
        assert torch.equal(leaf.grad, direct[name]), name
    assert torch.equal(h0.grad, direct["dh0"])
    want = oracle.gdn_dual_bwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), 4, inp.do,
                               inp.don, h0=inp.h0, dh_final=to_np(dhf), flags=flags)
    for name, leaf in zip(names, leaves):
        assert rel_rms(to_np(leaf.grad), want[name]) <= TOL_BF16, name
    assert rel_rms(to_np(h0.grad), want["dh0"]) <= TOL_BF16


def test_autograd_without_h0_and_unused_outputs(dev):
    import torch
    import gated_deltanet_dual_amd as g
    from gated_deltanet_dual_amd.autograd import gdn_dual
    inp = wl.gdn_inputs([100, 37], [20, 0], 2, 128, 128, 4, seed=83, with_grads=True)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    leaves = [t.clone().requires_grad_(True) for t in fwd_args(inp, dev)]
    o, on, hf = gdn_dual(vl, *leaves, 4)
    do = to_dev(inp.do, dev, True)
    (o.float() * do.float()).sum().backward()   # o~ and h_final unused: zero output gradients
    want = oracle.gdn_dual_bwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), 4, inp.do,
                               np.zeros_like(inp.don))
    torch.cuda.synchronize()
    for name, leaf in zip(("dq", "dk", "dv", "dalpha", "dbeta"), leaves):
        assert rel_rms(to_np(leaf.grad), want[name]) <= TOL_BF16, name
    assert not torch.any(leaves[5].grad), "q~ cannot affect a loss on the clean outputs"


@pytest.mark.parametrize("stride,window", [(4, 0), (2, 4), (1, 2)])
def test_autograd_memory_modes(dev, stride, window):
    """Strided checkpoints and chunk windows through the autograd wrapper:
    the same gradients as the default mode, bit for bit, and less device
    memory held between the forward and the backward."""
    import torch
    import gated_deltanet_dual_amd as g
    from gated_deltanet_dual_amd.autograd import gdn_dual
    inp = wl.gdn_inputs([300, 64, 200], [32, 0, 48], 2, 128, 128, 4, seed=90 + stride, with_h0=True,
                        with_grads=True)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    do, don = to_dev(inp.do, dev, True), to_dev(inp.don, dev, True)

    def run(**kw):
        leaves = [t.clone().requires_grad_(True) for t in fwd_args(inp, dev)]
        h0 = to_dev(inp.h0, dev).requires_grad_(True)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated(dev)
        o, on, hf = gdn_dual(vl, *leaves, 4, h0=h0, **kw)
        torch.cuda.synchronize()
        held = torch.cuda.memory_allocated(dev) - before
        ((o.float() * do.float()).sum() + (on.float() * don.float()).sum() + hf.sum()).backward()
        torch.cuda.synchronize()
        return [t.grad for t in leaves] + [h0.grad], held

    ref, held_ref = run()
    got, held = run(ckpt_stride=stride, window=window)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    assert held < held_ref, (held, held_ref)
