"""Pins for the fp64 oracle: every check here is fixed by the mathematics of
the pages' definitions, not by the oracle itself.

Sources: "FLARE: Diffusion for Hybrid Language Model" (papernotes.org notes),
Overall framework (prompt clean, response in blocks of B) and Key designs items
2 (gated delta rule, noisy block inheritance, block-end read), 3 (ShortConv
guard, document packing) and 4 (serving EVAL / COMMIT).
"""
import json
import os

import numpy as np
import pytest

import oracle
from brute import chunked, unrolled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def rand_case(rng, doc_lens, prompts, H, dk, dv, norm=True, h0=True):
    T = int(sum(doc_lens))
    cu = np.concatenate([[0], np.cumsum(doc_lens)]).astype(np.int32)

    def qk(d):
        x = rng.standard_normal((T, H, d))
        return x / np.linalg.norm(x, axis=-1, keepdims=True) if norm else x

    c = dict(
        cu=cu, pl=np.asarray(prompts, np.int32),
        q=qk(dk), k=qk(dk), v=rng.standard_normal((T, H, dv)),
        a=rng.uniform(0.5, 1.0, (T, H)), b=rng.uniform(0.05, 1.0, (T, H)),
        qn=qk(dk), kn=qk(dk), vn=rng.standard_normal((T, H, dv)),
        an=rng.uniform(0.5, 1.0, (T, H)), bn=rng.uniform(0.05, 1.0, (T, H)),
        h0=rng.standard_normal((len(doc_lens), H, dk, dv)) if h0 else None,
    )
    return c


def fwd(c, B, scale=0.0, flags=0, **over):
    d = dict(c)
    d.update(over)
    return oracle.gdn_dual_fwd(d["cu"], d["pl"], d["q"], d["k"], d["v"], d["a"], d["b"],
                               d["qn"], d["kn"], d["vn"], d["an"], d["bn"], B,
                               h0=d["h0"], scale=scale, flags=flags)


# --------------------------------------------------------------------------
# hand-worked examples
# --------------------------------------------------------------------------

def test_golden_hand_gdn():
    g = json.load(open(GOLDEN))["gdn_d2"]
    ex = lambda key: np.asarray(g[key], float)[:, None, :]
    gate = lambda key: np.asarray(g[key], float)[:, None]
    o, on, hf = oracle.gdn_dual_fwd(g["cu_seqlens"], g["prompt_lens"], ex("q"), ex("k"), ex("v"),
                                    gate("alpha"), gate("beta"), ex("qn"), ex("kn"), ex("vn"),
                                    gate("alpha_n"), gate("beta_n"), g["block_size"],
                                    scale=g["scale"])
    np.testing.assert_array_equal(o[:, 0], np.asarray(g["expect_o"], float))
    np.testing.assert_array_equal(on[:, 0], np.asarray(g["expect_on"], float))
    np.testing.assert_array_equal(hf[0, 0], np.asarray(g["expect_h_final"], float))


def test_golden_hand_shortconv():
    g = json.load(open(GOLDEN))["shortconv_w2"]
    y, yn = oracle.shortconv_dual(g["cu_seqlens"], g["prompt_lens"], g["block_size"],
                                  g["x"], g["xn"], g["weight"])
    np.testing.assert_array_equal(y, np.asarray(g["expect_y"], float))
    np.testing.assert_array_equal(yn, np.asarray(g["expect_yn"], float))


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------

def test_beta_zero_closed_form():
    """beta = 0 everywhere: S_t = (prod a) S_0, o_t = s (prod a) S_0^T q_t and the
    noisy read is s (prod of clean a up to the boundary)(prod of the block's a~) S_0^T q~."""
    rng = np.random.default_rng(10)
    c = rand_case(rng, [11], [3], 2, 4, 3)
    c["b"] = np.zeros_like(c["b"])
    c["bn"] = np.zeros_like(c["bn"])
    B = 3
    s = 1 / np.sqrt(4)
    o, on, hf = fwd(c, B)
    ca = np.cumprod(c["a"], axis=0)
    for h in range(2):
        S0 = c["h0"][0, h]
        for t in range(11):
            np.testing.assert_allclose(o[t, h], s * ca[t, h] * S0.T @ c["q"][t, h], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(hf[0, h], ca[-1, h] * S0, rtol=1e-13)
        for t0 in range(3, 11, B):
            e = min(t0 + B, 11)
            f = ca[t0 - 1, h] * np.prod(c["an"][t0:e, h])
            for l in range(t0, e):
                np.testing.assert_allclose(on[l, h], s * f * S0.T @ c["qn"][l, h], rtol=1e-13, atol=1e-14)
        np.testing.assert_array_equal(on[:3, h], 0.0)


def test_exact_retrieval_orthonormal_keys():
    """a = 1, b = 1, orthonormal keys, S_0 = 0: reading with q = k_j returns the
    latest value written under key j exactly; rewriting a key overwrites it."""
    rng = np.random.default_rng(11)
    d = 6
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm.T  # rows orthonormal
    order = [0, 1, 2, 1, 3, 0, 4, 5, 2]
    n = len(order)
    k = keys[order][:, None, :]
    v = rng.standard_normal((n, 1, 5))
    q = k.copy()
    ones = np.ones((n, 1))
    o, on, hf = oracle.gdn_dual_fwd([0, n], [n], q, k, v, ones, ones, q, k, v, ones, ones, 2,
                                    scale=1.0)
    latest = {}
    for t, j in enumerate(order):
        latest[j] = v[t, 0]
        np.testing.assert_allclose(o[t, 0], v[t, 0], atol=1e-12)
    for j, val in latest.items():
        np.testing.assert_allclose(hf[0, 0].T @ keys[j], val, atol=1e-12)


def test_lms_step_identities():
    """For a unit key: k^T S_t = a (1-b) k^T S_{t-1} + b v^T and
    (I - k k^T) S_t = a (I - k k^T) S_{t-1}.  States are read as h_final of
    prefix documents packed into one batch."""
    rng = np.random.default_rng(12)
    n, H, dk, dv = 9, 1, 5, 4
    base = rand_case(rng, [n], [n], H, dk, dv, h0=False)
    # pack every prefix length 1..n as its own document with the same content
    lens = list(range(1, n + 1))
    idx = np.concatenate([np.arange(L) for L in lens])
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    sub = {key: (base[key][idx] if key not in ("cu", "pl", "h0") else None) for key in base}
    _, _, hf = oracle.gdn_dual_fwd(cu, lens, sub["q"], sub["k"], sub["v"], sub["a"], sub["b"],
                                   sub["qn"], sub["kn"], sub["vn"], sub["an"], sub["bn"], 2)
    for t in range(1, n):
        kt = base["k"][t, 0]
        a, b = base["a"][t, 0], base["b"][t, 0]
        Sp, St = hf[t - 1, 0], hf[t, 0]
        np.testing.assert_allclose(kt @ St, a * (1 - b) * (kt @ Sp) + b * base["v"][t, 0], atol=1e-12)
        Pk = np.eye(dk) - np.outer(kt, kt)
        np.testing.assert_allclose(Pk @ St, a * Pk @ Sp, atol=1e-12)


# --------------------------------------------------------------------------
# brute force and the chunked algebra
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,P,B,dk,dv", [(12, 4, 3, 4, 3), (9, 0, 2, 3, 5), (7, 7, 2, 3, 3),
                                         (10, 2, 4, 5, 2), (6, 0, 8, 3, 4), (1, 0, 1, 2, 2)])
def test_unrolled_products(n, P, B, dk, dv):
    rng = np.random.default_rng(100 + n * 7 + P)
    c = rand_case(rng, [n], [P], 2, dk, dv)
    s = 1 / np.sqrt(dk)
    o, on, hf = fwd(c, B)
    for h in range(2):
        bo, bon, bS = unrolled(*(c[x][:, h] for x in ("q", "k", "v", "a", "b", "qn", "kn", "vn", "an", "bn")),
                               P, B, c["h0"][0, h], s)
        np.testing.assert_allclose(o[:, h], bo, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(on[:, h], bon, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(hf[0, h], bS, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("n,P,B,C", [(40, 8, 4, 16), (37, 12, 4, 8), (64, 0, 8, 32), (20, 20, 4, 8),
                                     (33, 4, 1, 4), (70, 16, 16, 16)])
def test_chunked_algebra_matches(n, P, B, C):
    rng = np.random.default_rng(200 + n + P + B + C)
    dk, dv = 6, 5
    c = rand_case(rng, [n], [P], 1, dk, dv)
    s = 0.37
    o, on, hf = fwd(c, B, scale=s)
    co, con, cS = chunked(*(c[x][:, 0] for x in ("q", "k", "v", "a", "b", "qn", "kn", "vn", "an", "bn")),
                          P, B, c["h0"][0, 0], s, C)
    np.testing.assert_allclose(o[:, 0], co, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(on[:, 0], con, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(hf[0, 0], cS, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------
# invariants of the dual stream
# --------------------------------------------------------------------------

def test_linearity_in_values_and_state():
    rng = np.random.default_rng(13)
    c1 = rand_case(rng, [10, 7], [2, 0], 2, 4, 3)
    c2 = rand_case(rng, [10, 7], [2, 0], 2, 4, 3)
    mix = dict(c1)
    for key in ("v", "vn", "h0"):
        mix[key] = 2.0 * c1[key] - 3.0 * c2[key]
    r1, r2, rm = fwd(c1, 2), fwd(dict(c1, v=c2["v"], vn=c2["vn"], h0=c2["h0"]), 2), fwd(mix, 2)
    for x1, x2, xm in zip(r1, r2, rm):
        np.testing.assert_allclose(xm, 2.0 * x1 - 3.0 * x2, rtol=1e-10, atol=1e-11)


def test_noisy_equal_clean_reads_block_end():
    """noisy inputs == clean inputs: on_l = s S_e^T q_l for every l of the block,
    so in particular on = o at the block end."""
    rng = np.random.default_rng(14)
    n, P, B, dk, dv = 23, 7, 4, 4, 3  # P not aligned: the oracle accepts any P
    c = rand_case(rng, [n], [P], 1, dk, dv)
    c["qn"], c["kn"], c["vn"], c["an"], c["bn"] = c["q"], c["k"], c["v"], c["a"], c["b"]
    o, on, _ = fwd(c, B)
    s = 1 / np.sqrt(dk)
    for t0 in range(P, n, B):
        e = min(t0 + B, n)
        np.testing.assert_allclose(on[e - 1], o[e - 1], rtol=1e-12, atol=1e-13)
        # S_e from a prefix document
        _, _, hf = oracle.gdn_dual_fwd([0, e], [e], *(c[x][:e] for x in ("q", "k", "v", "a", "b",
                                                                       "qn", "kn", "vn", "an", "bn")),
                                       B, h0=c["h0"])
        for l in range(t0, e):
            np.testing.assert_allclose(on[l, 0], s * hf[0, 0].T @ c["q"][l, 0], rtol=1e-12, atol=1e-13)


def test_block_size_one_is_one_noisy_step():
    rng = np.random.default_rng(15)
    n, P, dk, dv = 9, 3, 4, 4
    c = rand_case(rng, [n], [P], 1, dk, dv)
    o, on, _ = fwd(c, 1, scale=1.0)
    for l in range(P, n):
        _, _, hf = oracle.gdn_dual_fwd([0, l], [l], *(c[x][:l] for x in ("q", "k", "v", "a", "b",
                                                                       "qn", "kn", "vn", "an", "bn")),
                                       1, h0=c["h0"])
        S = hf[0, 0]
        kk, a, b = c["kn"][l, 0], c["an"][l, 0], c["bn"][l, 0]
        S1 = a * (S - b * np.outer(kk, kk @ S)) + b * np.outer(kk, c["vn"][l, 0])
        np.testing.assert_allclose(on[l, 0], S1.T @ c["qn"][l, 0], rtol=1e-12, atol=1e-13)


def test_block_covering_response_starts_from_prompt_state():
    rng = np.random.default_rng(16)
    n, P, dk, dv = 14, 5, 3, 4
    c = rand_case(rng, [n], [P], 1, dk, dv)
    _, on_big, _ = fwd(c, 64)
    _, _, hP = oracle.gdn_dual_fwd([0, P], [P], *(c[x][:P] for x in ("q", "k", "v", "a", "b",
                                                                   "qn", "kn", "vn", "an", "bn")),
                                   4, h0=c["h0"])
    S = hP[0, 0].copy()
    for l in range(P, n):
        kk, a, b = c["kn"][l, 0], c["an"][l, 0], c["bn"][l, 0]
        S = a * (S - b * np.outer(kk, kk @ S)) + b * np.outer(kk, c["vn"][l, 0])
    for l in range(P, n):
        np.testing.assert_allclose(on_big[l, 0], S.T @ c["qn"][l, 0] / np.sqrt(dk), rtol=1e-12, atol=1e-13)


def test_clean_outputs_ignore_noisy_inputs_and_block_locality():
    rng = np.random.default_rng(17)
    n, P, B = 26, 6, 4
    c = rand_case(rng, [n], [P], 2, 4, 4)
    o0, on0, hf0 = fwd(c, B)
    c2 = dict(c)
    c2["qn"] = c["qn"].copy()
    c2["vn"] = c["vn"].copy()
    c2["an"] = c["an"].copy()
    # perturb noisy block 2 (tokens P+8 .. P+11) only
    blk = slice(P + 2 * B, P + 3 * B)
    c2["vn"][blk] += 1.0
    c2["an"][blk] *= 0.9
    c2["qn"][blk] *= -1.0
    o1, on1, hf1 = fwd(c2, B)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(hf0, hf1)
    changed = np.any(on0 != on1, axis=(1, 2))
    assert changed[blk].all()
    changed[blk] = False
    assert not changed.any()


def test_packing_equals_separate_documents():
    rng = np.random.default_rng(18)
    lens, prompts = [9, 0, 13, 4], [4, 0, 0, 4]
    c = rand_case(rng, lens, prompts, 2, 4, 3)
    o, on, hf = fwd(c, 2)
    cu = c["cu"]
    for i, (L, P) in enumerate(zip(lens, prompts)):
        sl = slice(cu[i], cu[i + 1])
        sub = {x: c[x][sl] for x in ("q", "k", "v", "a", "b", "qn", "kn", "vn", "an", "bn")}
        oi, oni, hfi = oracle.gdn_dual_fwd([0, L], [P], *(sub[x] for x in ("q", "k", "v", "a", "b",
                                                                         "qn", "kn", "vn", "an", "bn")),
                                           2, h0=c["h0"][i:i + 1])
        np.testing.assert_array_equal(o[sl], oi)
        np.testing.assert_array_equal(on[sl], oni)
        np.testing.assert_array_equal(hf[i], hfi[0])


def test_l2norm_flag_equals_prenormalised():
    rng = np.random.default_rng(19)
    c = rand_case(rng, [12, 8], [4, 2], 2, 5, 3, norm=False)
    nrm = lambda x: x / np.sqrt((x * x).sum(-1, keepdims=True) + 1e-6)
    r_flag = fwd(c, 2, flags=oracle.FLAG_QK_L2NORM)
    r_pre = fwd(dict(c, q=nrm(c["q"]), k=nrm(c["k"]), qn=nrm(c["qn"]), kn=nrm(c["kn"])), 2)
    for x, y in zip(r_flag, r_pre):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-14)


def test_oracle_rejects_bad_lengths():
    rng = np.random.default_rng(20)
    c = rand_case(rng, [5], [2], 1, 2, 2)
    with pytest.raises(ValueError):
        fwd(dict(c, pl=np.array([6], np.int32)), 2)


# --------------------------------------------------------------------------
# serving step
# --------------------------------------------------------------------------

def test_block_step_eval_and_commit_match_dual_forward():
    """EVAL from pool state S_P equals the dual forward's noisy block output;
    COMMIT equals the clean forward over the block and its final state; EVAL
    leaves the pool untouched and is repeatable."""
    rng = np.random.default_rng(21)
    H, dk, dv, B, P = 2, 4, 3, 4, 8
    c = rand_case(rng, [P + B], [P], H, dk, dv)
    o, on, hf = fwd(c, B)
    _, _, hP = oracle.gdn_dual_fwd([0, P], [P], *(c[x][:P] for x in ("q", "k", "v", "a", "b",
                                                                   "qn", "kn", "vn", "an", "bn")),
                                   B, h0=c["h0"])
    n_slots = 5
    pool = rng.standard_normal((n_slots, H, dk, dv))
    pool[3] = hP[0]
    before = pool.copy()
    blk = slice(P, P + B)
    as_req = lambda x: x[blk][None]
    oe = oracle.block_step([3], pool, as_req(c["qn"]), as_req(c["kn"]), as_req(c["vn"]),
                           as_req(c["an"]), as_req(c["bn"]), oracle.EVAL)
    np.testing.assert_array_equal(pool, before)
    np.testing.assert_allclose(oe[0], on[blk], rtol=1e-12, atol=1e-13)
    oe2 = oracle.block_step([3], pool, as_req(c["qn"]), as_req(c["kn"]), as_req(c["vn"]),
                            as_req(c["an"]), as_req(c["bn"]), oracle.EVAL)
    np.testing.assert_array_equal(oe, oe2)
    oc = oracle.block_step([3], pool, as_req(c["q"]), as_req(c["k"]), as_req(c["v"]),
                           as_req(c["a"]), as_req(c["b"]), oracle.COMMIT)
    np.testing.assert_allclose(oc[0], o[blk], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(pool[3], hf[0], rtol=1e-12, atol=1e-13)
    other = [i for i in range(n_slots) if i != 3]
    np.testing.assert_array_equal(pool[other], before[other])


def test_block_step_rejects_duplicate_slots():
    pool = np.zeros((4, 1, 2, 2))
    x = np.zeros((2, 1, 1, 2))
    g = np.ones((2, 1, 1))
    with pytest.raises(ValueError):
        oracle.block_step([1, 1], pool, x, x, x, g, g, oracle.EVAL)
    with pytest.raises(ValueError):
        oracle.block_step([1, 4], pool, x, x, x, g, g, oracle.EVAL)


# --------------------------------------------------------------------------
# ShortConv
# --------------------------------------------------------------------------

def test_shortconv_clean_is_library_convolution():
    """The clean stream is a per-document causal depthwise convolution:
    numpy.convolve of the document with the reversed kernel, first n outputs."""
    rng = np.random.default_rng(30)
    lens, prompts, B, C, W = [11, 3, 17], [4, 0, 8], 4, 5, 4
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((T, C))
    xn = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    y, yn = oracle.shortconv_dual(cu, prompts, B, x, xn, w)
    for i in range(len(lens)):
        for ch in range(C):
            ref = np.convolve(x[cu[i]:cu[i + 1], ch], w[ch, ::-1])[:lens[i]]
            np.testing.assert_allclose(y[cu[i]:cu[i + 1], ch], ref, rtol=1e-13, atol=1e-13)
    # identical streams -> identical outputs on response rows, zero prompt rows
    y2, yn2 = oracle.shortconv_dual(cu, prompts, B, x, x, w)
    for i in range(len(lens)):
        r0 = cu[i] + prompts[i]
        np.testing.assert_array_equal(yn2[cu[i]:r0], 0.0)
        np.testing.assert_allclose(yn2[r0:cu[i + 1]], y2[r0:cu[i + 1]], rtol=1e-14)


def test_shortconv_position_tags():
    """x^c[t] = t, x^n[t] = -t-1 and a one-hot weight at lag j: the output names
    the source (sign) and the position (magnitude) every tap read."""
    lens, prompts, B, W = [13, 9], [5, 0], 4, 4
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    pos = np.concatenate([np.arange(L) for L in lens]).astype(float)
    x = pos[:, None] + 1000.0 * np.repeat(np.arange(2), lens)[:, None]  # doc id in the thousands
    xn = -x - 1.0
    for lag in range(W):
        w = np.zeros((1, W))
        w[0, W - 1 - lag] = 1.0
        y, yn = oracle.shortconv_dual(cu, prompts, B, x, xn, w)
        for i, (L, P) in enumerate(zip(lens, prompts)):
            for t in range(L):
                g = cu[i] + t
                m = t - lag
                exp_c = 0.0 if m < 0 else x[cu[i] + m, 0]
                assert y[g, 0] == exp_c
                if t < P:
                    assert yn[g, 0] == 0.0
                else:
                    blk = P + ((t - P) // B) * B
                    exp_n = 0.0 if m < 0 else (x[cu[i] + m, 0] if m < blk else xn[cu[i] + m, 0])
                    assert yn[g, 0] == exp_n


def test_shortconv_bias_and_silu():
    rng = np.random.default_rng(31)
    lens, prompts = [8], [4]
    x = rng.standard_normal((8, 3))
    w = rng.standard_normal((3, 4))
    bias = rng.standard_normal(3)
    y0, yn0 = oracle.shortconv_dual([0, 8], prompts, 4, x, x, w)
    y1, yn1 = oracle.shortconv_dual([0, 8], prompts, 4, x, x, w, bias=bias, activation=1)
    z = y0 + bias
    np.testing.assert_allclose(y1, z / (1 + np.exp(-z)), rtol=1e-13)
    zn = yn0[4:] + bias
    np.testing.assert_allclose(yn1[4:], zn / (1 + np.exp(-zn)), rtol=1e-13)
    np.testing.assert_array_equal(yn1[:4], 0.0)


def test_shortconv_silu_and_bias_special_values():
    """SiLU and the bias pinned by values the sigmoid fixes in closed form:
    sigma(ln 3) = 3/4 and sigma(-ln 3) = 1/4, so silu(ln 3) = (3/4) ln 3 and
    silu(-ln 3) = -(1/4) ln 3; silu(0) = 0; silu(x) -> x for large x.  A
    one-hot current tap passes x through; zero taps leave only the bias, on
    every row including the first rows of a document."""
    l3 = np.log(3.0)
    vals = np.array([0.0, l3, -l3, 40.0])
    x = np.repeat(vals[:, None], 2, axis=1)  # one document of 4 tokens, 2 channels
    w = np.zeros((2, 4))
    w[:, 3] = 1.0  # tap W - 1 multiplies the current token
    y, _ = oracle.shortconv_dual([0, 4], [4], 4, x, x, w, activation=1)
    want = np.array([0.0, 0.75 * l3, -0.25 * l3, 40.0])
    np.testing.assert_allclose(y[:, 0], want, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(y[:, 1], want, rtol=1e-15, atol=1e-15)
    # zero taps: the activated bias alone, on every row
    yb, _ = oracle.shortconv_dual([0, 4], [4], 4, x, x, np.zeros((2, 4)), bias=np.array([l3, -l3]),
                                  activation=1)
    np.testing.assert_allclose(yb[:, 0], 0.75 * l3, rtol=1e-15)
    np.testing.assert_allclose(yb[:, 1], -0.25 * l3, rtol=1e-15)
    # without the activation the bias is a plain shift
    y0, _ = oracle.shortconv_dual([0, 4], [4], 4, x, x, w)
    y1, _ = oracle.shortconv_dual([0, 4], [4], 4, x, x, w, bias=np.array([0.5, -2.0]))
    np.testing.assert_allclose(y1 - y0, np.tile([0.5, -2.0], (4, 1)), rtol=0, atol=1e-15)
