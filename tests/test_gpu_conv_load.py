"""The dual-stream forward with the layer's ShortConv in its loads
(flare_gdn_dual_fwd_conv) through the C ABI.

"FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes), Key
designs items 2-3: the dual ShortConv in front of the GDN layer, fused into
it.  The kernels form every q, k, v row from the raw projections with the
ShortConv's own arithmetic and rounding, so the result must equal the two-step
path -- the standalone prologue (no L2 step) writing the rows, then the plain
forward reading them -- bit for bit; with the q/k L2 flag the factors come from
the same sums as the factor pass.  The two-step path is itself held to the
oracle elsewhere; here the fused path is also checked against the oracle's
composition of the same two steps."""
import numpy as np
import pytest

import oracle
from gated_deltanet_dual_amd import workloads as wl
from gpu_util import TOL_BF16, rel_rms, to_dev, to_np

pytestmark = pytest.mark.gpu

# documents crossing chunk boundaries, prompts at 0, at chunk starts and
# mid-chunk, empty and sub-chunk documents (prompts rounded down to B below)
LENS = [200, 45, 0, 97, 31, 130, 5, 64]
PROMPTS = [12, 0, 0, 64, 28, 100, 4, 36]


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


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def draw(seed, lens, prompts, H, W):
    """Projections (bf16), conv weights, gates; the noisy projections' prompt
    rows hold huge values, which must never reach an output."""
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    C = H * 128
    xs = [wl.round_bf16(rng.standard_normal((T, C)).astype(np.float32)) for _ in range(3)]
    xns = [wl.round_bf16(rng.standard_normal((T, C)).astype(np.float32)) for _ in range(3)]
    cu = _cu(lens)
    for x in xns:
        for i, p in enumerate(prompts):
            x[cu[i]:cu[i] + p] = 3.0e38
    ws = [rng.uniform(-0.5, 0.5, (C, W)).astype(np.float32) for _ in range(3)]
    gates = []
    for _ in range(2):
        gates.append(np.exp(-0.1 * np.log1p(np.exp(rng.standard_normal((T, H))))).astype(np.float32))
        gates.append((1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32))
    h0 = (rng.standard_normal((len(lens), H, 128, 128)) / 11.3).astype(np.float32)
    return xs, xns, ws, gates, h0


def two_step(g, vl, B, gx, gxn, gw, gates, h0, act, flags, **kw):
    """The standalone prologue (no L2 step), then the plain forward."""
    T, C = gx[0].shape
    H = C // 128
    ys, yns = g.qkv_prologue(vl, B, 128, gx, gxn, gw, activation=act, qk_l2norm=False)
    hv = lambda t: t.view(T, H, 128)
    return g.gdn_dual_fwd(vl, hv(ys[0]), hv(ys[1]), hv(ys[2]), gates[0], gates[1], hv(yns[0]), hv(yns[1]),
                          hv(yns[2]), gates[2], gates[3], B, h0=h0, flags=flags, want_ckpt=True, **kw)


def ckpt_rows_equal(ck, ref, cu, stride=1):
    import torch
    for i in range(len(cu) - 1):
        n = cu[i + 1] - cu[i]
        for c in range(0, (n + 31) // 32, stride):
            s = cu[i] // (32 * stride) + i + c // stride
            assert torch.equal(ck[s], ref[s]), (i, c)


@pytest.mark.parametrize("W,act,flags,B", [(4, 1, 0, 4), (4, 1, 1, 4), (4, 0, 1, 8), (3, 1, 0, 1), (2, 0, 1, 32),
                                           (1, 1, 1, 16), (4, 1, 1, 2)])
def test_conv_load_equals_prologue_then_forward(g, dev, W, act, flags, B):
    import torch
    prompts = [min(n, (p // B) * B) for n, p in zip(LENS, PROMPTS)]
    H = 2
    xs, xns, ws, gates, h0 = draw(900 + 10 * W + B, LENS, prompts, H, W)
    vl = g.Varlen(_cu(LENS), prompts, dev)
    gx, gxn = [to_dev(x, dev, True) for x in xs], [to_dev(x, dev, True) for x in xns]
    gw, gg, gh0 = [to_dev(w, dev) for w in ws], [to_dev(a, dev) for a in gates], to_dev(h0, dev)
    ref = two_step(g, vl, B, gx, gxn, gw, gg, gh0, act, flags)
    got = g.gdn_dual_fwd_conv(vl, gx, gxn, gw, *gg, B, activation=act, h0=gh0, flags=flags, want_ckpt=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "on", "h_final"), got[:3], ref[:3]):
        assert torch.equal(a, b), name
    ckpt_rows_equal(got[3], ref[3], _cu(LENS))


@pytest.mark.parametrize("flags", [0, 1])
def test_conv_load_against_oracle(g, dev, flags):
    """Against the oracle's composition: its prologue (fp64), rounded to bf16
    where the pipeline stores rows, then its forward."""
    import torch
    B, H, W = 4, 2, 4
    prompts = [min(n, (p // B) * B) for n, p in zip(LENS, PROMPTS)]
    xs, xns, ws, gates, h0 = draw(950 + flags, LENS, prompts, H, W)
    cu = _cu(LENS)
    vl = g.Varlen(cu, prompts, dev)
    o, on, hf, _ = g.gdn_dual_fwd_conv(vl, [to_dev(x, dev, True) for x in xs], [to_dev(x, dev, True) for x in xns],
                                       [to_dev(w, dev) for w in ws], *[to_dev(a, dev) for a in gates], B,
                                       activation=1, h0=to_dev(h0, dev), flags=flags)
    torch.cuda.synchronize()
    r16 = lambda y: wl.round_bf16(np.asarray(y, np.float32)).astype(np.float64)
    rys, ryns = oracle.qkv_prologue(cu, prompts, B, 128, xs, xns, ws, activation=1, l2=False)
    T = int(cu[-1])
    rh = lambda y: r16(y).reshape(T, H, 128)
    ro, ron, rhf = oracle.gdn_dual_fwd(cu, prompts, *map(rh, rys), gates[0], gates[1], *map(rh, ryns), gates[2],
                                       gates[3], B, h0=h0, flags=flags)
    assert rel_rms(to_np(o), ro) <= TOL_BF16
    assert rel_rms(to_np(on), ron) <= TOL_BF16
    assert rel_rms(to_np(hf), rhf) <= TOL_BF16


def test_conv_load_windows_and_stride(g, dev):
    """Windows of 2 chunks and stride-2 checkpoints: the same bits as one pass."""
    import torch
    B, H, W = 4, 2, 4
    prompts = [min(n, (p // B) * B) for n, p in zip(LENS, PROMPTS)]
    xs, xns, ws, gates, h0 = draw(970, LENS, prompts, H, W)
    vl = g.Varlen(_cu(LENS), prompts, dev)
    args = ([to_dev(x, dev, True) for x in xs], [to_dev(x, dev, True) for x in xns], [to_dev(w, dev) for w in ws],
            *[to_dev(a, dev) for a in gates], B)
    ref = g.gdn_dual_fwd_conv(vl, *args, h0=to_dev(h0, dev), flags=1, want_ckpt=True, ckpt_stride=2)
    got = g.gdn_dual_fwd_conv(vl, *args, h0=to_dev(h0, dev), flags=1, want_ckpt=True, ckpt_stride=2, window=2)
    torch.cuda.synchronize()
    for a, b in zip(got[:3], ref[:3]):
        assert torch.equal(a, b)
    ckpt_rows_equal(got[3], ref[3], _cu(LENS), 2)


def test_conv_load_packed_full_size(g, dev):
    """The packed row (32768 tokens, 8 documents, 32 heads x 128, W = 4, SiLU,
    q/k L2 flag): every head bit-identical to the two-step path."""
    import torch
    p = wl.packed_conv(round_io=False)
    B, H, d = p["block_size"], p["H"], p["d"]
    T = int(p["cu_seqlens"][-1])
    C = H * d
    vl = g.Varlen(p["cu_seqlens"], p["prompt_lens"], dev)
    x = to_dev(p["x"], dev, True)
    xn = to_dev(p["xn"], dev, True)
    w = to_dev(p["weight"], dev)
    gx = [x[:, s * C:(s + 1) * C].contiguous() for s in range(3)]
    gxn = [xn[:, s * C:(s + 1) * C].contiguous() for s in range(3)]
    gw = [w[s * C:(s + 1) * C].contiguous() for s in range(3)]
    del x, xn
    gg = [to_dev(p[k], dev) for k in ("alpha", "beta", "alpha_n", "beta_n")]
    ref = two_step(g, vl, B, gx, gxn, gw, gg, None, 1, g.QK_L2NORM, want_h_final=True)
    got = g.gdn_dual_fwd_conv(vl, gx, gxn, gw, *gg, B, activation=1, flags=g.QK_L2NORM)
    torch.cuda.synchronize()
    for name, a, b in zip(("o", "on", "h_final"), got[:3], ref[:3]):
        assert torch.equal(a, b), name
