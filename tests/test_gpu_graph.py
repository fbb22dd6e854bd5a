"""The serving cycle (four EVALs and a COMMIT through the C-ABI binding)
captured once as a HIP graph (torch.cuda.CUDAGraph on the library's stream)
and replayed: every replay, with eager work and synchronisations in between
and the pool restored from its initial copy before each, reproduces the eager
cycle bit for bit (the same kernels on the same inputs are deterministic).
The step launches no memset, so nothing in the graph is a memset node.
"""
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


@pytest.mark.parametrize("d,bf16", [(128, True), (16, False)])
def test_serving_cycle_graph_replays_match_eager(g, dev, d, bf16):
    import torch
    rng = np.random.default_rng(100 + d)
    R, B, H, n_slots = 12, 4, 2, 20
    slots = to_dev(rng.permutation(n_slots)[:R].astype(np.int32), dev)
    pool0 = to_dev((rng.standard_normal((n_slots, H, d, d)) / np.sqrt(d)).astype(np.float32), dev)
    rnd = wl.round_bf16 if bf16 else (lambda a: a)

    def block():
        q = rnd(rng.standard_normal((R, B, H, d)).astype(np.float32))
        k = rng.standard_normal((R, B, H, d)).astype(np.float32)
        k = rnd((k / np.linalg.norm(k, axis=3, keepdims=True)).astype(np.float32))
        v = rnd(rng.standard_normal((R, B, H, d)).astype(np.float32))
        a = rng.uniform(0.85, 1.0, (R, B, H)).astype(np.float32)
        b = rng.uniform(0.1, 0.9, (R, B, H)).astype(np.float32)
        return [to_dev(q, dev, bf16), to_dev(k, dev, bf16), to_dev(v, dev, bf16), to_dev(a, dev), to_dev(b, dev)]

    blocks = [block() for _ in range(5)]
    dt = torch.bfloat16 if bf16 else torch.float32
    outs = [torch.empty((R, B, H, d), dtype=dt, device=dev) for _ in range(5)]
    pool = pool0.clone()

    def cycle():
        for e in range(4):
            g.block_step(slots, pool, *blocks[e], g.EVAL, o=outs[e])
        g.block_step(slots, pool, *blocks[4], g.COMMIT, o=outs[4])

    # eager reference
    cycle()
    torch.cuda.synchronize()
    want_o = [o.clone() for o in outs]
    want_pool = pool.clone()

    # warm up on a side stream, then capture
    pool.copy_(pool0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cycle()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    pool.copy_(pool0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        cycle()
    torch.cuda.synchronize()

    for rep in range(3):
        for o in outs:
            o.zero_()
        pool.copy_(pool0)
        junk = torch.randn(1 << 20, device=dev).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for e in range(5):
            assert torch.equal(outs[e], want_o[e]), (rep, e)
        assert torch.equal(pool, want_pool), rep
