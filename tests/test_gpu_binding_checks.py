"""On the GPU: argument mistakes that would read or write device memory out
of bounds, or silently misread a view, raise FlareError in the binding before
any launch; the same call with the mistake fixed runs."""
import pytest

from gated_deltanet_dual_amd import workloads as wl
from gpu_util import fwd_args, to_dev

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


def test_forward_and_backward_argument_mistakes(g, dev):
    import torch
    inp = wl.gdn_inputs([70, 33], [16, 0], 2, 128, 128, 4, seed=5, with_grads=True)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    args = fwd_args(inp, dev)
    bad = list(args)
    bad[3] = args[3].to(torch.bfloat16)                      # bf16 gates
    with pytest.raises(g.FlareError, match="alpha: dtype"):
        g.gdn_dual_fwd(vl, *bad, 4)
    bad = list(args)
    bad[0] = args[0].transpose(1, 2).contiguous().transpose(1, 2)  # a non-contiguous view
    with pytest.raises(g.FlareError, match="contiguous"):
        g.gdn_dual_fwd(vl, *bad, 4)
    short = g.Varlen([0, 70, 100], [16, 0], dev)             # T disagrees with cu_seqlens
    with pytest.raises(g.FlareError, match="cu_seqlens"):
        g.gdn_dual_fwd(short, *args, 4)
    with pytest.raises(g.FlareError, match="h0: shape"):
        g.gdn_dual_fwd(vl, *args, 4, h0=torch.zeros((2, 2, 128, 64), device=dev))
    nslots = g.ckpt_slots(vl, 2, 128, 4, g.BF16)
    with pytest.raises(g.FlareError, match="ckpt holds"):
        g.gdn_dual_fwd(vl, *args, 4, ckpt=torch.empty((nslots - 1, 2, 128, 128), device=dev))
    with pytest.raises(g.FlareError, match="workspace holds"):
        g.gdn_dual_fwd(vl, *args, 4, workspace=torch.empty(1024, dtype=torch.uint8, device=dev))
    o, on, hf, ck = g.gdn_dual_fwd(vl, *args, 4, want_ckpt=True)
    do, don = to_dev(inp.do, dev, True), to_dev(inp.don, dev, True)
    with pytest.raises(g.FlareError, match="d_o: shape"):
        g.gdn_dual_bwd(vl, *args, 4, ck, do[:, :1], don)
    with pytest.raises(g.FlareError, match="ckpt holds"):
        g.gdn_dual_bwd(vl, *args, 4, ck[:-1], do, don)
    gr = g.gdn_dual_bwd(vl, *args, 4, ck, do, don)
    gr["dalpha"] = torch.empty((inp.T, 2), dtype=torch.bfloat16, device=dev)
    with pytest.raises(g.FlareError, match="dalpha: dtype"):
        g.gdn_dual_bwd(vl, *args, 4, ck, do, don, out=gr)
    torch.cuda.synchronize()


def test_serving_argument_mistakes(g, dev):
    import torch
    s = wl.serving(seed=3, n_req=4, H=2, d=128, n_slots=6, n_evals=1)
    pool = to_dev(s.pool, dev)
    slot = to_dev(s.slot_idx, dev)
    q, k, v, a, b = s.evals[0]
    X = [to_dev(q, dev, True), to_dev(k, dev, True), to_dev(v, dev, True), to_dev(a, dev), to_dev(b, dev)]
    with pytest.raises(g.FlareError, match="pool: shape"):
        g.block_step(slot, pool[:, :1].contiguous(), *X, g.EVAL)            # pool with another H
    with pytest.raises(g.FlareError, match="slot_idx: dtype"):
        g.block_step(slot.long(), pool, *X, g.EVAL)
    with pytest.raises(g.FlareError, match="o: shape"):
        g.block_step(slot, pool, *X, g.EVAL, o=torch.empty((4, 2, 2, 128), dtype=torch.bfloat16, device=dev))
    g.block_step(slot, pool, *X, g.EVAL)
    torch.cuda.synchronize()
