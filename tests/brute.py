"""Independent fp64 numpy formulations used to pin the oracle.

Neither function re-types the oracle's token loop:

* ``unrolled`` builds the transition matrices M_t = a_t (I - b_t k_t k_t^T) as
  explicit dense matrices and forms every state from the closed product
  S_t = M_t...M_1 S_0 + sum_j M_t...M_{j+1} b_j k_j v_j^T (the gated delta rule
  of the FLARE notes, Key designs item 2, unrolled).
* ``chunked`` is the chunk-parallel (WY / UT-transform) rewrite of the same
  recurrence: per chunk of C tokens, T = (I + A)^-1 with
  A_ij = (G_i/G_j) b_j k_i.k_j (j < i), U = T (V - diag(G) K S_c), outputs from
  S_c plus a causally masked intra-chunk term, and the noisy block-boundary
  reads S_p^T x formed from S_c with the mask j < p instead of materialising S_p.
  This is the algebra the GPU kernels implement; pinning it to the oracle at
  1e-12 checks the algebra before any kernel exists.
"""
from __future__ import annotations

import numpy as np


def _boundaries(n, P, B):
    return [t for t in range(P, n, B)]


def unrolled(q, k, v, a, b, qn, kn, vn, an, bn, P, B, S0, s):
    """One document, one head.  Returns (o, on, S_n)."""
    n, dk = k.shape
    dv = v.shape[1]
    I = np.eye(dk)
    M = [a[t] * (I - b[t] * np.outer(k[t], k[t])) for t in range(n)]

    def prod(mats):
        out = I.copy()
        for m in mats:          # mats in application order
            out = m @ out
        return out

    def state(tcount):
        """clean state after tcount tokens, from the unrolled product form"""
        S = prod(M[:tcount]) @ S0
        for j in range(tcount):
            S = S + prod(M[j + 1:tcount]) @ (b[j] * np.outer(k[j], v[j]))
        return S

    o = np.zeros((n, dv))
    for t in range(n):
        o[t] = s * state(t + 1).T @ q[t]
    on = np.zeros((n, dv))
    Mn = [an[t] * (I - bn[t] * np.outer(kn[t], kn[t])) for t in range(n)]
    for t0 in _boundaries(n, P, B):
        e = min(t0 + B, n)
        Sp = state(t0)
        Se = prod(Mn[t0:e]) @ Sp
        for j in range(t0, e):
            Se = Se + prod(Mn[j + 1:e]) @ (bn[j] * np.outer(kn[j], vn[j]))
        for l in range(t0, e):
            on[l] = s * Se.T @ qn[l]
    return o, on, state(n)


def chunked(q, k, v, a, b, qn, kn, vn, an, bn, P, B, S0, s, C):
    """Chunk-parallel form; requires P % B == 0 and C % B == 0."""
    assert P % B == 0 and C % B == 0
    n, dk = k.shape
    dv = v.shape[1]
    S = S0.copy()
    o = np.zeros((n, dv))
    on = np.zeros((n, dv))
    for c0 in range(0, n, C):
        c1 = min(c0 + C, n)
        L = c1 - c0
        K, Q, V, bt = k[c0:c1], q[c0:c1], v[c0:c1], b[c0:c1]
        g = np.cumsum(np.log(a[c0:c1]))
        G = np.exp(g)
        E = np.exp(g[:, None] - g[None, :])
        A = np.tril(E * (K @ K.T) * bt[None, :], -1)
        Tm = np.linalg.inv(np.eye(L) + A)
        U = Tm @ (V - G[:, None] * (K @ S))
        o[c0:c1] = s * (G[:, None] * (Q @ S) + (np.tril(Q @ K.T * E) * bt[None, :]) @ U)
        for t0 in _boundaries(n, P, B):
            if not (c0 <= t0 < c1):
                continue
            e = min(t0 + B, n)
            p = t0 - c0
            Gp = np.exp(g[p - 1]) if p > 0 else 1.0
            Qn, Kn, Vn = qn[t0:e], kn[t0:e], vn[t0:e]
            w = (Gp / G[:p]) * bt[:p]
            rq = Gp * (Qn @ S) + ((Qn @ K[:p].T) * w[None, :]) @ U[:p]
            rk = Gp * (Kn @ S) + ((Kn @ K[:p].T) * w[None, :]) @ U[:p]
            gn = np.cumsum(np.log(an[t0:e]))
            Gn = np.exp(gn)
            En = np.exp(gn[:, None] - gn[None, :])
            An = np.tril(En * (Kn @ Kn.T) * bn[t0:e][None, :], -1)
            Un = np.linalg.inv(np.eye(e - t0) + An) @ (Vn - Gn[:, None] * rk)
            wn = (Gn[-1] / Gn) * bn[t0:e]
            on[t0:e] = s * (Gn[-1] * rq + ((Qn @ Kn.T) * wn[None, :]) @ Un)
        S = G[-1] * S + K.T @ (((bt * G[-1] / G))[:, None] * U)
    return o, on, S
