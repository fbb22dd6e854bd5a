"""fp64 CPU oracle for the dual-stream Gated DeltaNet layer -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It wraps ``flare_oracle.c`` (plain C, fp64, pthreads over
independent (document, head) or (request, head) units) through ctypes on numpy
float64 arrays.  It never imports the HIP library and the HIP library never
imports it.

What each entry computes, with its source:

* ``gdn_dual_fwd`` -- the gated delta rule of "FLARE: Diffusion for Hybrid
  Language Model" (papernotes.org notes, Key designs item 2) run token by token
  over every document; each noisy block copies the clean boundary state, applies
  its own noisy updates and all of its positions read the block-end state.
* ``gdn_dual_bwd`` -- reverse mode of the same recurrence, the noisy block-start
  adjoint added to the clean adjoint at the block boundary (same item).
* ``block_step`` -- serving EVAL (no pool write) and COMMIT (causal replay that
  writes the pool), Key designs item 4.
* ``gdn_verify`` / ``gdn_scatter`` -- AR-Trust (same page, Key designs item
  4): the clean stream verifies K drafted tokens in one causal pass from the
  pool state, keeping the state after every token as a candidate; once r
  tokens are accepted, candidate r is copied into the pool.
* ``block_step_conv`` / ``conv_cache_fill`` -- the serving step with the
  ShortConv in front: each request keeps its last W-1 clean projection rows,
  so a block's taps before its start read that clean history and taps inside
  read the block itself; the prefill fills the history from the prompt.
* ``shortconv_dual`` -- the dual-source causal ShortConv, Key designs item 3.
* ``shortconv_dual_bwd`` -- its reverse mode (parity pinned by finite
  differences and the adjoint identity in the CPU tests).
* ``qkv_prologue`` / ``qkv_prologue_bwd`` -- the GDN layer's input prologue:
  the ShortConv above on each of the q, k, v projections of both streams,
  optionally SiLU, then (a reading: the pages do not mention it) q and k
  divided per (token, head) by sqrt(sum x^2 + 1e-6); and its reverse mode.
  Plain numpy around the C ShortConv.

Parity pins (closed forms, brute force, invariants, finite differences and a
hand-worked example) are in the CPU tests; see ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "flare_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

FLAG_QK_L2NORM = 1
EVAL, COMMIT = 0, 1


_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")
# FLARE_ORACLE_SANITIZED=1 loads the AddressSanitizer + UndefinedBehaviorSanitizer
# build instead (the process must preload libasan; see tests/test_sanitizers.py)
_SANITIZED = os.environ.get("FLARE_ORACLE_SANITIZED") == "1"


def build(sanitized: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (always recompiles); with sanitized,
    ``liboracle_san.so`` built with -fsanitize=address,undefined."""
    out = _LIB_SAN if sanitized else _LIB
    tmp = out + ".tmp%d" % os.getpid()
    flags = ["-O2"]
    if sanitized:
        flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                 "-fno-sanitize-recover=all"]
    cmd = ["gcc"] + flags + ["-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC",
                             "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _LIB_SAN if _SANITIZED else _LIB
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        build(sanitized=_SANITIZED)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, f64 = ctypes.c_int, ctypes.c_double
    lib.oracle_gdn_dual_fwd.argtypes = [i32, P, P, i32, i32, i32, i32, f64, i32] + [P] * 14 + [i32]
    lib.oracle_gdn_dual_fwd.restype = i32
    lib.oracle_gdn_dual_bwd.argtypes = [i32, P, P, i32, i32, i32, i32, f64, i32] + [P] * 25 + [i32]
    lib.oracle_gdn_dual_bwd.restype = i32
    lib.oracle_block_step.argtypes = [i32, P, P, i32, i32, i32, i32, i32, f64] + [P] * 6 + [i32, i32]
    lib.oracle_block_step.restype = i32
    lib.oracle_gdn_verify.argtypes = [i32, P, P, i32, i32, i32, i32, i32, f64] + [P] * 7 + [i32]
    lib.oracle_gdn_verify.restype = i32
    lib.oracle_shortconv_dual.argtypes = [i32, P, P, i32, i32, i32, P, P, P, P, i32, P, P, i32]
    lib.oracle_shortconv_dual.restype = i32
    lib.oracle_shortconv_dual_bwd.argtypes = [i32, P, P, i32, i32, i32, P, P, P, P, i32, P, P, P, P, P, P, i32]
    lib.oracle_shortconv_dual_bwd.restype = i32
    lib.oracle_default_threads.argtypes = []
    lib.oracle_default_threads.restype = i32
    _lib = lib
    return lib


def default_threads() -> int:
    return int(_load().oracle_default_threads())


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _p(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _check(rc, name):
    if rc != 0:
        raise ValueError("%s: invalid arguments (status %d)" % (name, rc))


def gdn_dual_fwd(cu_seqlens, prompt_lens, q, k, v, alpha, beta, qn, kn, vn,
                 alpha_n, beta_n, block_size, h0=None, scale=0.0, flags=0,
                 threads=0):
    """Dual-stream forward.  q,k,qn,kn: [T,H,dk]; v,vn: [T,H,dv];
    gates [T,H]; h0 [N,H,dk,dv] or None.  Returns (o, on, h_final)."""
    cu, pl = _i32(cu_seqlens), _i32(prompt_lens)
    q, k, v, a, b = map(_f64, (q, k, v, alpha, beta))
    qn, kn, vn, an, bn = map(_f64, (qn, kn, vn, alpha_n, beta_n))
    h0 = _f64(h0)
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(pl)
    o = np.zeros((T, H, dv))
    on = np.zeros((T, H, dv))
    hf = np.zeros((N, H, dk, dv))
    rc = _load().oracle_gdn_dual_fwd(N, _p(cu), _p(pl), H, dk, dv, int(block_size),
                                     float(scale), int(flags), _p(q), _p(k), _p(v),
                                     _p(a), _p(b), _p(qn), _p(kn), _p(vn), _p(an),
                                     _p(bn), _p(h0), _p(o), _p(on), _p(hf), int(threads))
    _check(rc, "gdn_dual_fwd")
    return o, on, hf


def gdn_dual_bwd(cu_seqlens, prompt_lens, q, k, v, alpha, beta, qn, kn, vn,
                 alpha_n, beta_n, block_size, do, don, h0=None, dh_final=None,
                 scale=0.0, flags=0, threads=0):
    """Reverse mode.  Returns a dict with dq, dk, dv, dalpha, dbeta, dqn, dkn,
    dvn, dalpha_n, dbeta_n, dh0."""
    cu, pl = _i32(cu_seqlens), _i32(prompt_lens)
    q, k, v, a, b = map(_f64, (q, k, v, alpha, beta))
    qn, kn, vn, an, bn = map(_f64, (qn, kn, vn, alpha_n, beta_n))
    h0, do, don, dhf = _f64(h0), _f64(do), _f64(don), _f64(dh_final)
    T, H, dk = q.shape
    dv = v.shape[2]
    N = len(pl)
    out = {
        "dq": np.zeros((T, H, dk)), "dk": np.zeros((T, H, dk)), "dv": np.zeros((T, H, dv)),
        "dalpha": np.zeros((T, H)), "dbeta": np.zeros((T, H)),
        "dqn": np.zeros((T, H, dk)), "dkn": np.zeros((T, H, dk)), "dvn": np.zeros((T, H, dv)),
        "dalpha_n": np.zeros((T, H)), "dbeta_n": np.zeros((T, H)),
        "dh0": np.zeros((N, H, dk, dv)),
    }
    rc = _load().oracle_gdn_dual_bwd(
        N, _p(cu), _p(pl), H, dk, dv, int(block_size), float(scale), int(flags),
        _p(q), _p(k), _p(v), _p(a), _p(b), _p(qn), _p(kn), _p(vn), _p(an), _p(bn),
        _p(h0), _p(do), _p(don), _p(dhf),
        _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dalpha"]), _p(out["dbeta"]),
        _p(out["dqn"]), _p(out["dkn"]), _p(out["dvn"]), _p(out["dalpha_n"]),
        _p(out["dbeta_n"]), _p(out["dh0"]), int(threads))
    _check(rc, "gdn_dual_bwd")
    return out


def block_step(slot_idx, pool, q, k, v, alpha, beta, mode, scale=0.0, threads=0):
    """Serving step.  pool [n_slots,H,dk,dv] is modified in place for COMMIT;
    q,k [R,B,H,dk], v [R,B,H,dv], gates [R,B,H].  Returns o [R,B,H,dv]."""
    slot = _i32(slot_idx)
    if not (isinstance(pool, np.ndarray) and pool.dtype == np.float64 and pool.flags.c_contiguous):
        raise TypeError("pool must be a C-contiguous float64 array (updated in place)")
    q, k, v, a, b = map(_f64, (q, k, v, alpha, beta))
    R, B, H, dk = q.shape
    dv = v.shape[3]
    o = np.zeros((R, B, H, dv))
    rc = _load().oracle_block_step(R, _p(slot), _p(pool), pool.shape[0], H, dk, dv, B,
                                   float(scale), _p(q), _p(k), _p(v), _p(a), _p(b),
                                   _p(o), int(mode), int(threads))
    _check(rc, "block_step")
    return o


def gdn_verify(slot_idx, pool, q, k, v, alpha, beta, scale=0.0, threads=0):
    """AR-Trust verify: the clean causal pass over K drafted tokens per request
    from its pool state.  q,k [R,K,H,dk], v [R,K,H,dv], gates [R,K,H].
    Returns (o [R,K,H,dv], cand [R,K,H,dk,dv]); the pool is not modified."""
    slot = _i32(slot_idx)
    pool = _f64(pool)
    q, k, v, a, b = map(_f64, (q, k, v, alpha, beta))
    R, K, H, dk = q.shape
    dv = v.shape[3]
    o = np.zeros((R, K, H, dv))
    cand = np.zeros((R, K, H, dk, dv))
    rc = _load().oracle_gdn_verify(R, _p(slot), _p(pool), pool.shape[0], H, dk, dv, K, float(scale),
                                   _p(q), _p(k), _p(v), _p(a), _p(b), _p(o), _p(cand), int(threads))
    _check(rc, "gdn_verify")
    return o, cand


def gdn_scatter(slot_idx, accepted, cand, pool):
    """AR-Trust rollback: for each request with r = accepted count clamped to
    [0, K], r >= 1 writes candidate r (the state after r tokens) into its pool
    slot; r = 0 leaves the slot as it was.  pool is updated in place."""
    K = cand.shape[1]
    for i, sl in enumerate(np.asarray(slot_idx)):
        r = min(max(int(accepted[i]), 0), K)
        if r >= 1:
            pool[sl] = cand[i, r - 1]
    return pool


def gdn_commit_prefix(slot_idx, pool, q, k, v, alpha, beta, accepted, scale=0.0):
    """AR-Trust rollback by replay: for each request, the COMMIT of its first
    r drafted tokens (r = accepted count clamped to [0, K]) into its pool slot
    (the serving step's causal replay, Key designs item 4); r = 0 leaves the
    slot.  pool is updated in place.  Returns the causal outputs of the
    replayed tokens, zero past r."""
    q, k, v, a, b = map(_f64, (q, k, v, alpha, beta))
    R, K = q.shape[:2]
    o = np.zeros(v.shape)
    for i, sl in enumerate(np.asarray(slot_idx)):
        r = min(max(int(accepted[i]), 0), K)
        if r == 0:
            continue
        part = lambda x: np.ascontiguousarray(x[i:i + 1, :r])
        o[i, :r] = block_step([0], pool[sl:sl + 1], part(q), part(k), part(v), part(a), part(b), COMMIT,
                              scale=scale)[0]
    return o


def shortconv_dual(cu_seqlens, prompt_lens, block_size, x, xn, weight,
                   bias=None, activation=0, threads=0):
    """x, xn [T,C]; weight [C,W]; bias [C] or None.  Returns (y, yn)."""
    cu, pl = _i32(cu_seqlens), _i32(prompt_lens)
    x, xn, w, bias = _f64(x), _f64(xn), _f64(weight), _f64(bias)
    T, C = x.shape
    W = w.shape[1]
    y = np.zeros((T, C))
    yn = np.zeros((T, C))
    rc = _load().oracle_shortconv_dual(len(pl), _p(cu), _p(pl), int(block_size), C, W,
                                       _p(x), _p(xn), _p(w), _p(bias), int(activation),
                                       _p(y), _p(yn), int(threads))
    _check(rc, "shortconv_dual")
    return y, yn


def shortconv_dual_bwd(cu_seqlens, prompt_lens, block_size, x, xn, weight, dy, dyn,
                       bias=None, activation=0, threads=0):
    """Reverse mode of shortconv_dual: x, xn, dy, dyn [T,C]; weight [C,W];
    bias [C] or None.  Returns (dx, dxn, dweight, dbias); dxn's prompt rows are
    0 and dyn's prompt rows are ignored."""
    cu, pl = _i32(cu_seqlens), _i32(prompt_lens)
    x, xn, w, bias = _f64(x), _f64(xn), _f64(weight), _f64(bias)
    dy, dyn = _f64(dy), _f64(dyn)
    T, C = x.shape
    W = w.shape[1]
    dx = np.zeros((T, C))
    dxn = np.zeros((T, C))
    dw = np.zeros((C, W))
    db = np.zeros(C)
    rc = _load().oracle_shortconv_dual_bwd(len(pl), _p(cu), _p(pl), int(block_size), C, W,
                                           _p(x), _p(xn), _p(w), _p(bias), int(activation),
                                           _p(dy), _p(dyn), _p(dx), _p(dxn), _p(dw), _p(db),
                                           int(threads))
    _check(rc, "shortconv_dual_bwd")
    return dx, dxn, dw, db


L2_EPS = 1e-6


def _l2_heads(y, d):
    """Divide every (token, head) row of d values by sqrt(sum y^2 + eps)."""
    T = y.shape[0]
    r = y.reshape(T, -1, d)
    n = np.sqrt(np.sum(r * r, axis=2, keepdims=True) + L2_EPS)
    return (r / n).reshape(y.shape)


def _l2_heads_bwd(y, dyhat, d):
    """Gradient w.r.t. y of sum(dyhat * y / n), n = sqrt(|y|^2 + eps) per row:
    dyhat / n - y (y . dyhat) / n^3."""
    T = y.shape[0]
    r = y.reshape(T, -1, d)
    g = dyhat.reshape(T, -1, d)
    n = np.sqrt(np.sum(r * r, axis=2, keepdims=True) + L2_EPS)
    dot = np.sum(r * g, axis=2, keepdims=True)
    return (g / n - r * dot / n ** 3).reshape(y.shape)


def qkv_prologue(cu_seqlens, prompt_lens, block_size, head_dim, xs, xns, weights, activation=0, l2=True,
                 threads=0):
    """ShortConv -> optional SiLU -> per-head L2 norm of q and k.
    xs, xns: the clean and noisy (q, k, v) projections, each [T, H*head_dim];
    weights: their conv weights, each [H*head_dim, W].  Returns (ys, yns), the
    GDN-ready (q, k, v) of both streams (noisy prompt rows 0)."""
    ys, yns = [], []
    for sec in range(3):
        y, yn = shortconv_dual(cu_seqlens, prompt_lens, block_size, xs[sec], xns[sec], weights[sec],
                               activation=activation, threads=threads)
        if l2 and sec < 2:
            y, yn = _l2_heads(y, head_dim), _l2_heads(yn, head_dim)
        ys.append(y)
        yns.append(yn)
    return ys, yns


def qkv_prologue_bwd(cu_seqlens, prompt_lens, block_size, head_dim, xs, xns, weights, dys, dyns,
                     activation=0, l2=True, threads=0):
    """Reverse mode of qkv_prologue: dys, dyns are the gradients of its
    outputs (noisy prompt rows ignored).  Returns (dxs, dxns, dws)."""
    dxs, dxns, dws = [], [], []
    for sec in range(3):
        dy, dyn = _f64(dys[sec]), _f64(dyns[sec])
        if l2 and sec < 2:
            y, yn = shortconv_dual(cu_seqlens, prompt_lens, block_size, xs[sec], xns[sec], weights[sec],
                                   activation=activation, threads=threads)
            dy, dyn = _l2_heads_bwd(y, dy, head_dim), _l2_heads_bwd(yn, dyn, head_dim)
        dx, dxn, dw, _ = shortconv_dual_bwd(cu_seqlens, prompt_lens, block_size, xs[sec], xns[sec],
                                            weights[sec], dy, dyn, activation=activation, threads=threads)
        dxs.append(dx)
        dxns.append(dxn)
        dws.append(dw)
    return dxs, dxns, dws


def conv_cache_fill(cu_seqlens, xs, width, doc_slot, cache):
    """The clean history of each document after a prefill: cache[slot_i][j, s]
    = xs[s][end_i - (W-1) + j] (zero before the document start).  cache:
    [n_slots, W-1, 3, C], updated in place."""
    W1 = width - 1
    for i, sl in enumerate(doc_slot):
        a, e = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
        for j in range(W1):
            t = e - W1 + j
            for sec in range(3):
                cache[sl, j, sec] = xs[sec][t] if t >= a else 0.0
    return cache


def block_step_conv(slot_idx, pool, cache, head_dim, xs, weights, alpha, beta, mode, activation=0, l2=True,
                    scale=0.0):
    """Serving step whose q, k, v come from raw projections xs (three
    [R, B, H*d]) through the ShortConv: request r's block is preceded by its
    clean history cache[slot_r] ([W-1, 3, H*d]) -- a one-document batch whose
    prompt is the history and whose one block is the drafted / fixed block.
    EVAL reads the block as the noisy stream (outputs at the block end), COMMIT
    as the clean stream and then keeps the last W-1 clean rows as the new
    history.  pool and cache are updated in place for COMMIT."""
    xs = [_f64(x) for x in xs]
    R, B, C = xs[0].shape
    W1 = cache.shape[1]
    H = C // head_dim
    q, k, v = (np.zeros((R, B, H, head_dim)) for _ in range(3))
    for r, sl in enumerate(slot_idx):
        n = W1 + B
        hist = [cache[sl, :, sec] for sec in range(3)]
        blk = [xs[sec][r] for sec in range(3)]
        if mode == EVAL:
            x = [np.concatenate([hist[sec], np.zeros((B, C))]) for sec in range(3)]
            xn = [np.concatenate([np.zeros((W1, C)), blk[sec]]) for sec in range(3)]
        else:
            x = [np.concatenate([hist[sec], blk[sec]]) for sec in range(3)]
            xn = x
        ys, yns = qkv_prologue([0, n], [W1], B, head_dim, x, xn, weights, activation=activation, l2=l2)
        out = yns if mode == EVAL else ys
        for sec, dst in enumerate((q, k, v)):
            dst[r] = out[sec][W1:].reshape(B, H, head_dim)
    o = block_step(slot_idx, pool, q, k, v, alpha, beta, EVAL if mode == EVAL else COMMIT, scale=scale)
    if mode != EVAL:
        for r, sl in enumerate(slot_idx):
            full = [np.concatenate([cache[sl, :, sec], xs[sec][r]]) for sec in range(3)]
            for sec in range(3):
                cache[sl, :, sec] = full[sec][B:]
    return o
