"""flare_qkv_prologue_bwd_noalloc (the allocation-free variant for callers
that cannot allocate: its weight-gradient partials live in the library's
static device scratch) against flare_qkv_prologue_bwd with a caller
workspace, through the C ABI: bit-identical results on two calls in a row,
the second on a smaller batch, so nothing of the first call's partials may
leak into the second; and a batch whose partials exceed the scratch is
refused before anything is launched."""
import numpy as np
import pytest

from gated_deltanet_dual_amd import workloads as wl
from gpu_util import to_dev

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


def batch(g, dev, lens, prompts, H, d, W, seed):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    vl = g.Varlen(cu, prompts, dev)
    mk = lambda: to_dev(wl.round_bf16(rng.standard_normal((T, H * d)).astype(np.float32)), dev, True)
    xs, xns, dys, dyns = [mk() for _ in range(3)], [mk() for _ in range(3)], [mk() for _ in range(3)], \
        [mk() for _ in range(3)]
    ws = [to_dev(rng.uniform(-0.5, 0.5, (H * d, W)).astype(np.float32), dev) for _ in range(3)]
    return vl, xs, xns, ws, dys, dyns


def outputs(torch, xs, W, dev):
    T, C = xs[0].shape
    return ([torch.empty_like(x) for x in xs], [torch.empty_like(x) for x in xs],
            [torch.empty((C, W), dtype=torch.float32, device=dev) for _ in range(3)])


def test_noalloc_matches_workspace_entry_point(g, dev):
    import torch
    lens, prompts = wl.packed_doc_lengths(32768, 8, 4, seed=3)
    cases = [
        # the packed training row: 32768 tokens, 8 documents, 32 heads x 128, W = 4, SiLU
        (list(lens), list(prompts), 32, 128, 4, 1),
        # then a smaller ragged batch (its partials cover a fraction of the first call's)
        ([37, 0, 70, 5, 300], [12, 0, 20, 4, 100], 2, 128, 3, 0),
    ]
    for i, (lens, prompts, H, d, W, act) in enumerate(cases):
        vl, xs, xns, ws, dys, dyns = batch(g, dev, lens, prompts, H, d, W, seed=50 + i)
        want = g.qkv_prologue_bwd(vl, 4, d, xs, xns, ws, dys, dyns, activation=act)
        got = g.qkv_prologue_bwd_noalloc(vl, 4, d, xs, xns, ws, dys, dyns, outputs(torch, xs, W, dev),
                                         activation=act)
        torch.cuda.synchronize()
        for a, b in zip(sum(map(list, want), []), sum(map(list, got), [])):
            assert torch.equal(a, b), (i, "the no-alloc results differ from the workspace entry point's")


def test_noalloc_refuses_batches_beyond_the_scratch(g, dev):
    import torch
    H, d, W = 32, 128, 8
    T = 49152                     # 3 sections x 192 token blocks x 4096 channels x 9 partials x 4 B > 64 MiB
    vl = g.Varlen(np.array([0, T], np.int32), np.array([0], np.int32), dev)
    assert g.qkv_prologue_bwd_workspace_bytes(vl, 4, H, d, W) > g.noalloc_scratch_bytes()
    x = [torch.empty((T, H * d), dtype=torch.bfloat16, device=dev) for _ in range(3)]
    ws = [torch.zeros((H * d, W), dtype=torch.float32, device=dev) for _ in range(3)]
    out = ([torch.empty_like(t) for t in x], [torch.empty_like(t) for t in x],
           [torch.empty((H * d, W), dtype=torch.float32, device=dev) for _ in range(3)])
    with pytest.raises(g.FlareError, match="static scratch") as e:
        g.qkv_prologue_bwd_noalloc(vl, 4, d, x, x, ws, x, x, out)
    assert e.value.status == 5
