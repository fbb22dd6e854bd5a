"""GPU parity of flare_qkv_prologue and flare_qkv_prologue_bwd (the GDN layer's
fused input prologue: ShortConv on the q, k, v projections of both streams,
optional SiLU, per-head L2 norm of q and k) through the C-ABI binding, against
the fp64 oracle (oracle.qkv_prologue, oracle.qkv_prologue_bwd), and of the
whole training path built on it: prologue -> dual GDN forward (no flags) ->
dual GDN backward -> prologue reverse mode, against the oracle's composition.

  * ragged documents (an empty one, one shorter than the window, runs and
    256-token blocks crossed), widths 3, 4, 6, fp32 and bf16 io, head sizes
    16 and 128 (4 to 64 lanes per head in the in-wave L2 sums);
  * the packed row of 32768 tokens, 8 documents, 32 heads x 128 per
    projection, W=4, bf16, on two sampled heads per projection;
  * the training path at d=128, bf16, on ragged documents.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_dual_amd import workloads as wl
from gpu_util import TOL_BF16, TOL_F32, rel_rms, to_dev, to_np

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


LENS = [37, 0, 3, 70, 5, 96, 1, 90]
PROMPTS = [12, 0, 0, 20, 4, 32, 0, 40]


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def draw(seed, T, H, d, W, bf16):
    rng = np.random.default_rng(seed)
    rnd = wl.round_bf16 if bf16 else (lambda a: a)
    xs = [rnd(rng.standard_normal((T, H * d)).astype(np.float32)) for _ in range(3)]
    xns = [rnd(rng.standard_normal((T, H * d)).astype(np.float32)) for _ in range(3)]
    ws = [rng.uniform(-0.5, 0.5, (H * d, W)).astype(np.float32) for _ in range(3)]
    return xs, xns, ws


@pytest.mark.parametrize("W,H,d,act,bf16", [(4, 2, 16, 0, False), (3, 3, 16, 1, True), (4, 2, 128, 1, True),
                                            (6, 2, 128, 0, True), (4, 4, 32, 1, False)])
def test_prologue_forward_and_reverse(g, dev, W, H, d, act, bf16):
    import torch
    cu, B = _cu(LENS), 4
    T = int(cu[-1])
    xs, xns, ws = draw(40 + W + d, T, H, d, W, bf16)
    rng = np.random.default_rng(3)
    rnd = wl.round_bf16 if bf16 else (lambda a: a)
    dys = [rnd(rng.standard_normal((T, H * d)).astype(np.float32)) for _ in range(3)]
    dyns = [rnd(rng.standard_normal((T, H * d)).astype(np.float32)) for _ in range(3)]
    vl = g.Varlen(cu, PROMPTS, dev)
    up = lambda a: to_dev(a, dev, bf16)
    ys, yns = g.qkv_prologue(vl, B, d, [up(x) for x in xs], [up(x) for x in xns], [to_dev(w, dev) for w in ws],
                             activation=act)
    dxs, dxns, dws = g.qkv_prologue_bwd(vl, B, d, [up(x) for x in xs], [up(x) for x in xns],
                                        [to_dev(w, dev) for w in ws], [up(x) for x in dys], [up(x) for x in dyns],
                                        activation=act)
    torch.cuda.synchronize()
    rys, ryns = oracle.qkv_prologue(cu, PROMPTS, B, d, xs, xns, ws, activation=act)
    rdx, rdxn, rdw = oracle.qkv_prologue_bwd(cu, PROMPTS, B, d, xs, xns, ws, dys, dyns, activation=act)
    tol = TOL_BF16 if bf16 else TOL_F32
    for sec in range(3):
        assert rel_rms(to_np(ys[sec]), rys[sec]) <= tol, sec
        assert rel_rms(to_np(yns[sec]), ryns[sec]) <= tol, sec
        assert rel_rms(to_np(dxs[sec]), rdx[sec]) <= tol, sec
        assert rel_rms(to_np(dxns[sec]), rdxn[sec]) <= tol, sec
        assert rel_rms(to_np(dws[sec]), rdw[sec]) <= max(tol, TOL_F32), sec
        for i, p in enumerate(PROMPTS):
            assert not to_np(yns[sec])[cu[i]:cu[i] + p].any()
            assert not to_np(dxns[sec])[cu[i]:cu[i] + p].any()


def test_prologue_packed_full_size_sampled_heads(g, dev):
    """One packed row of 32768 tokens, 8 Dirichlet-split docs, q/k/v each
    32 heads x 128, W=4, bf16; the oracle checks heads 0 and 31 of each."""
    import torch
    p = wl.packed_conv()
    T, C3 = p["x"].shape
    C, d = C3 // 3, 128
    x, xn = to_dev(p["x"], dev, True), to_dev(p["xn"], dev, True)
    w = to_dev(p["weight"], dev)
    xs = [x[:, s * C:(s + 1) * C].contiguous() for s in range(3)]
    xns = [xn[:, s * C:(s + 1) * C].contiguous() for s in range(3)]
    ws = [w[s * C:(s + 1) * C].contiguous() for s in range(3)]
    vl = g.Varlen(p["cu_seqlens"], p["prompt_lens"], dev)
    rng = np.random.default_rng(12)
    dys = [wl.round_bf16(rng.standard_normal((T, C), dtype=np.float32)) for _ in range(3)]
    dyns = [wl.round_bf16(rng.standard_normal((T, C), dtype=np.float32)) for _ in range(3)]
    ys, yns = g.qkv_prologue(vl, p["block_size"], d, xs, xns, ws)
    dxs, dxns, dws = g.qkv_prologue_bwd(vl, p["block_size"], d, xs, xns, ws, [to_dev(a, dev, True) for a in dys],
                                        [to_dev(a, dev, True) for a in dyns])
    torch.cuda.synchronize()
    ch = np.r_[0:d, C - d:C]
    sub = lambda a, s: np.ascontiguousarray(a[:, s * C:(s + 1) * C][:, ch])
    rys, ryns = oracle.qkv_prologue(p["cu_seqlens"], p["prompt_lens"], p["block_size"], d,
                                    [sub(p["x"], s) for s in range(3)], [sub(p["xn"], s) for s in range(3)],
                                    [np.ascontiguousarray(p["weight"][s * C:(s + 1) * C][ch]) for s in range(3)])
    rdx, rdxn, rdw = oracle.qkv_prologue_bwd(
        p["cu_seqlens"], p["prompt_lens"], p["block_size"], d, [sub(p["x"], s) for s in range(3)],
        [sub(p["xn"], s) for s in range(3)],
        [np.ascontiguousarray(p["weight"][s * C:(s + 1) * C][ch]) for s in range(3)],
        [np.ascontiguousarray(a[:, ch]) for a in dys], [np.ascontiguousarray(a[:, ch]) for a in dyns])
    for sec in range(3):
        assert rel_rms(to_np(ys[sec][:, ch]), rys[sec]) <= TOL_BF16, sec
        assert rel_rms(to_np(yns[sec][:, ch]), ryns[sec]) <= TOL_BF16, sec
        assert rel_rms(to_np(dxs[sec][:, ch]), rdx[sec]) <= TOL_BF16, sec
        assert rel_rms(to_np(dxns[sec][:, ch]), rdxn[sec]) <= TOL_BF16, sec
        assert rel_rms(to_np(dws[sec][ch]), rdw[sec]) <= TOL_F32, sec


def test_training_path_prologue_gdn(g, dev):
    """prologue -> GDN forward (chunk-start states saved) -> GDN backward ->
    prologue reverse mode, bf16, d=128, ragged documents, SiLU, against the
    oracle's composition of the same four steps."""
    import torch
    lens, prompts, B, H, d, W = [100, 37, 0, 150, 9], [20, 4, 0, 52, 0], 4, 2, 128, 4
    cu = _cu(lens)
    T = int(cu[-1])
    xs, xns, ws = draw(77, T, H, d, W, True)
    rng = np.random.default_rng(78)
    a = np.exp(-0.1 * np.log1p(np.exp(rng.standard_normal((T, H))))).astype(np.float32)
    b = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    an = np.exp(-0.1 * np.log1p(np.exp(rng.standard_normal((T, H))))).astype(np.float32)
    bn = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    do = wl.round_bf16(rng.standard_normal((T, H, d)).astype(np.float32))
    don = wl.round_bf16(rng.standard_normal((T, H, d)).astype(np.float32))
    vl = g.Varlen(cu, prompts, dev)
    up = lambda x: to_dev(x, dev, True)
    gx, gxn, gw = [up(x) for x in xs], [up(x) for x in xns], [to_dev(w, dev) for w in ws]
    ys, yns = g.qkv_prologue(vl, B, d, gx, gxn, gw, activation=1)
    hv = lambda t: t.view(T, H, d)
    gates = [to_dev(u, dev) for u in (a, b, an, bn)]
    o, on, _, ckpt = g.gdn_dual_fwd(vl, hv(ys[0]), hv(ys[1]), hv(ys[2]), gates[0], gates[1], hv(yns[0]),
                                    hv(yns[1]), hv(yns[2]), gates[2], gates[3], B, want_ckpt=True)
    gr = g.gdn_dual_bwd(vl, hv(ys[0]), hv(ys[1]), hv(ys[2]), gates[0], gates[1], hv(yns[0]), hv(yns[1]),
                        hv(yns[2]), gates[2], gates[3], B, ckpt, up(do), up(don))
    flat = lambda t: t.reshape(T, H * d)
    dxs, dxns, dws = g.qkv_prologue_bwd(vl, B, d, gx, gxn, gw, [flat(gr[k]) for k in ("dq", "dk", "dv")],
                                        [flat(gr[k]) for k in ("dqn", "dkn", "dvn")], activation=1)
    torch.cuda.synchronize()
    # bf16 io: the pipeline stores the prologue outputs and the GDN gradients
    # as bf16 between its steps, so the oracle's composition rounds its own
    # fp64 values at the same two points
    r16 = lambda y: wl.round_bf16(np.asarray(y, np.float32)).astype(np.float64)
    rys, ryns = oracle.qkv_prologue(cu, prompts, B, d, xs, xns, ws, activation=1)
    rys, ryns = [r16(y) for y in rys], [r16(y) for y in ryns]
    rh = lambda y: y.reshape(T, H, d)
    ro, ron, _ = oracle.gdn_dual_fwd(cu, prompts, *map(rh, rys), a, b, *map(rh, ryns), an, bn, B)
    rg = oracle.gdn_dual_bwd(cu, prompts, *map(rh, rys), a, b, *map(rh, ryns), an, bn, B, do, don)
    rf = lambda y: r16(y.reshape(T, H * d))
    rdx, rdxn, rdw = oracle.qkv_prologue_bwd(cu, prompts, B, d, xs, xns, ws, [rf(rg[k]) for k in ("dq", "dk", "dv")],
                                             [rf(rg[k]) for k in ("dqn", "dkn", "dvn")], activation=1)
    assert rel_rms(to_np(o), ro) <= TOL_BF16
    assert rel_rms(to_np(on), ron) <= TOL_BF16
    for sec in range(3):
        assert rel_rms(to_np(dxs[sec]), rdx[sec]) <= TOL_BF16, sec
        assert rel_rms(to_np(dxns[sec]), rdxn[sec]) <= TOL_BF16, sec
        assert rel_rms(to_np(dws[sec]), rdw[sec]) <= TOL_BF16, sec
    for k in ("dalpha", "dbeta", "dalpha_n", "dbeta_n"):
        assert rel_rms(to_np(gr[k]), rg[k]) <= TOL_BF16, k
