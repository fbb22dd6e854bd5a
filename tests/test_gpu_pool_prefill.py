"""GPU parity of flare_gdn_dual_fwd_pool (prefill straight into serving-pool
slots) through the C-ABI binding, against the fp64 oracle's dual forward with
the same initial states:
  * bf16 io at d = 128 (the chunked path) and fp32 io at d = 16 (the fused
    per-document kernels), ragged documents including an empty one;
  * read_initial = 1 (documents continue from their slots' states, read before
    they are overwritten) and 0 (documents start from zero);
  * every slot that holds no document is bit-identical afterwards, and the
    pool then serves an EVAL like any other.
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


@pytest.mark.parametrize("d,io,read_initial", [(128, "bf16", True), (128, "bf16", False), (16, "f32", True),
                                               (16, "f32", False)])
def test_prefill_into_pool(g, dev, d, io, read_initial):
    import torch
    lens, prompts = [130, 0, 64, 97, 33], [32, 0, 64, 20, 4]
    H, B, n_slots = 2, 4, 9
    inp = wl.gdn_inputs(lens, prompts, H, d, d, B, seed=60 + d, io=io)
    rng = np.random.default_rng(61)
    pool = (rng.standard_normal((n_slots, H, d, d)) / np.sqrt(d)).astype(np.float32)
    slots = rng.permutation(n_slots)[:len(lens)].astype(np.int32)
    gpool = to_dev(pool, dev)
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    o, on = g.gdn_dual_fwd_pool(vl, *fwd_args(inp, dev), B, to_dev(slots, dev), gpool, read_initial=read_initial,
                                doc_slot_host=slots)
    torch.cuda.synchronize()
    h0 = pool[slots].astype(np.float64) if read_initial else None
    ro, ron, rhf = oracle.gdn_dual_fwd(inp.cu_seqlens, inp.prompt_lens, *inp.clean_args(), *inp.noisy_args(), B,
                                       h0=h0)
    tol = TOL_BF16 if io == "bf16" else TOL_F32
    assert rel_rms(to_np(o), ro) <= tol
    assert rel_rms(to_np(on), ron) <= tol
    got = gpool.cpu().numpy()
    assert rel_rms(got[slots], rhf) <= TOL_F32
    others = np.setdiff1d(np.arange(n_slots), slots)
    assert np.array_equal(got[others], pool[others])
    # the filled pool serves an EVAL (block-end reads of a fresh noisy block)
    blk = [rng.standard_normal((len(lens), B, H, d)).astype(np.float32) for _ in range(3)]
    blk = [wl.round_bf16(x) if io == "bf16" else x for x in blk]
    ga = rng.uniform(0.85, 1.0, (len(lens), B, H)).astype(np.float32)
    gb = rng.uniform(0.1, 0.9, (len(lens), B, H)).astype(np.float32)
    bf16 = io == "bf16"
    oe = g.block_step(to_dev(slots, dev), gpool, *(to_dev(x, dev, bf16) for x in blk), to_dev(ga, dev),
                      to_dev(gb, dev), g.EVAL, slot_idx_host=slots)
    torch.cuda.synchronize()
    roe = oracle.block_step(slots, got.astype(np.float64), *blk, ga, gb, oracle.EVAL)
    assert rel_rms(to_np(oe), roe) <= tol


def test_prefill_rejects_duplicate_slots(g, dev):
    inp = wl.gdn_inputs([40, 40], [8, 8], 1, 16, 16, 4, seed=62, io="f32")
    vl = g.Varlen(inp.cu_seqlens, inp.prompt_lens, dev)
    pool = to_dev(np.zeros((4, 1, 16, 16), np.float32), dev)
    with pytest.raises(g.FlareError):
        g.gdn_dual_fwd_pool(vl, *fwd_args(inp, dev), 4, to_dev(np.array([2, 2], np.int32), dev), pool,
                            doc_slot_host=[2, 2])
