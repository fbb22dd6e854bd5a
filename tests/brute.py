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


def chunked_backward(q, k, v, a, b, qn, kn, vn, an, bn, P, B, S0, s, C, do, don, dSn):
    """Reverse mode of ``chunked`` in the same chunk-parallel form (one
    document, one head).  A reverse scan carries dS (the adjoint of each chunk's
    start state) from chunk to chunk; within a chunk every gradient follows from
    matrix calculus on the chunk formulas:
      U = T rhs, T = (I + A)^-1      ->  d rhs = T^T dU,   dA = -d rhs U^T
      o = s(diag(G) Q S_c + Mo U)    ->  dU += s Mo^T dO, dQ += s diag(G) dO S_c^T, ...
    Gate gradients are collected per cumulative log-decay (gamma) and turned
    into d alpha by a reverse cumulative sum.  Returns the same dict as the
    oracle's reverse mode (without the batch axes)."""
    assert P % B == 0 and C % B == 0
    n, dk = k.shape
    dv = v.shape[1]
    # forward chunk states
    states = []
    S = S0.copy()
    for c0 in range(0, n, C):
        states.append(S.copy())
        c1 = min(c0 + C, n)
        K, V, bt = k[c0:c1], v[c0:c1], b[c0:c1]
        g = np.cumsum(np.log(a[c0:c1]))
        G = np.exp(g)
        E = np.exp(g[:, None] - g[None, :])
        A = np.tril(E * (K @ K.T) * bt[None, :], -1)
        Tm = np.linalg.inv(np.eye(c1 - c0) + A)
        U = Tm @ (V - G[:, None] * (K @ S))
        S = G[-1] * S + K.T @ ((bt * G[-1] / G)[:, None] * U)
    out = {x: np.zeros_like(y) for x, y in (("dq", q), ("dk", k), ("dv", v), ("dqn", qn), ("dkn", kn),
                                              ("dvn", vn))}
    dga = np.zeros(n)   # d/d log(alpha)
    dgan = np.zeros(n)
    dbeta = np.zeros(n)
    dbetan = np.zeros(n)
    dS = dSn.copy()     # adjoint of the state after the document
    starts = list(range(0, n, C))
    for ci in reversed(range(len(starts))):
        c0 = starts[ci]
        c1 = min(c0 + C, n)
        L = c1 - c0
        Sc = states[ci]
        K, Q, V, bt = k[c0:c1], q[c0:c1], v[c0:c1], b[c0:c1]
        g = np.cumsum(np.log(a[c0:c1]))
        G = np.exp(g)
        E = np.tril(np.exp(g[:, None] - g[None, :]))
        lower = np.tril(np.ones((L, L)), -1)
        GKK = K @ K.T
        A = GKK * E * lower * bt[None, :]
        Tm = np.linalg.inv(np.eye(L) + A)
        KS = K @ Sc
        rhs = V - G[:, None] * KS
        U = Tm @ rhs
        GQK = Q @ K.T
        Mo = GQK * E * bt[None, :]
        Dd = bt * G[-1] / G
        dO = do[c0:c1]
        dgam = np.zeros(L)      # d/d gamma_i (cumulative log alpha inside the chunk)
        dgamn = np.zeros(L)
        # ---- noisy blocks of this chunk
        tok = np.arange(c0, c1)
        resp = tok >= P
        pl = (np.arange(L) // B) * B         # chunk-local block start of each row
        dU = np.zeros_like(U)
        dSc = G[-1] * dS
        if resp.any():
            Qn, Kn, Vn, btn = qn[c0:c1], kn[c0:c1], vn[c0:c1], bn[c0:c1]
            gn = np.zeros(L)
            for s0 in range(0, L, B):
                gn[s0:s0 + B] = np.cumsum(np.log(an[c0 + s0:c0 + min(s0 + B, L)]))
            Gn = np.exp(gn)
            ge = np.array([gn[min(pl[i] + B, L) - 1] for i in range(L)])
            gp = np.array([g[pl[i] - 1] if pl[i] > 0 else 0.0 for i in range(L)])
            Gp = np.exp(gp)
            same = pl[:, None] == pl[None, :]
            maskq = (np.arange(L)[None, :] < pl[:, None]) & resp[:, None]
            Fq = np.where(maskq, np.exp(gp[:, None] - g[None, :]), 0.0)
            GQnK, GKnK = Qn @ K.T, Kn @ K.T
            Mq, Mk = GQnK * Fq * bt[None, :], GKnK * Fq * bt[None, :]
            En = np.where(same & resp[:, None], np.exp(gn[:, None] - gn[None, :]), 0.0)
            GKnKn = Kn @ Kn.T
            An = GKnKn * En * lower * btn[None, :]
            Tn = np.linalg.inv(np.eye(L) + An)
            Fe = np.where(same & resp[:, None], np.exp(ge[:, None] - gn[None, :]), 0.0)
            GQnKn = Qn @ Kn.T
            Mn = GQnKn * Fe * btn[None, :]
            QnS, KnS = Qn @ Sc, Kn @ Sc
            rq = Gp[:, None] * QnS + Mq @ U
            rk = Gp[:, None] * KnS + Mk @ U
            rhsn = Vn - Gn[:, None] * rk
            un = Tn @ rhsn
            dOn = np.where(resp[:, None], don[c0:c1], 0.0)
            # o~ = s (diag(Ge) rq + Mn un)
            drq = s * np.exp(ge)[:, None] * dOn
            dMn = s * dOn @ un.T
            dun = s * Mn.T @ dOn
            np.add.at(dgamn, [min(pl[i] + B, L) - 1 for i in range(L)], s * np.exp(ge) * (dOn * rq).sum(1))
            # un = Tn rhsn
            drhsn = Tn.T @ dun
            dAn = -drhsn @ un.T
            out["dvn"][c0:c1] = np.where(resp[:, None], drhsn, 0.0)
            # rhsn = Vn - diag(Gn) rk
            drk = -Gn[:, None] * drhsn
            dgamn += -Gn * (drhsn * rk).sum(1)
            # rq, rk
            dU += Mq.T @ drq + Mk.T @ drk
            dMq, dMk = drq @ U.T, drk @ U.T
            dSc += Qn.T @ (Gp[:, None] * drq) + Kn.T @ (Gp[:, None] * drk)
            dgp = Gp * ((drq * QnS).sum(1) + (drk * KnS).sum(1))
            dQn = Gp[:, None] * drq @ Sc.T
            dKn = Gp[:, None] * drk @ Sc.T
            # Gram gradients, noisy side
            for dM, M, F, X, Y, is_q in ((dMq, Mq, Fq, Qn, K, True), (dMk, Mk, Fq, Kn, K, False)):
                dG = dM * F * bt[None, :]
                if is_q:
                    dQn += dG @ K
                else:
                    dKn += dG @ K
                out["dk"][c0:c1] += dG.T @ X
                dbeta[c0:c1] += (dM * (X @ Y.T) * F).sum(0)
                dgp += (dM * M).sum(1)
                dgam -= (dM * M).sum(0)
            for i in range(L):
                if pl[i] > 0:
                    dgam[pl[i] - 1] += dgp[i]
            dGn = dMn * Fe * btn[None, :]
            dQn += dGn @ Kn
            dKn += dGn.T @ Qn
            dbetan[c0:c1] += (dMn * GQnKn * Fe).sum(0)
            for i in range(L):
                dgamn[min(pl[i] + B, L) - 1] += (dMn[i] * Mn[i]).sum()
            dgamn -= (dMn * Mn).sum(0)
            EnL = En * lower
            dGAn = dAn * EnL * btn[None, :]
            dKn += dGAn @ Kn + dGAn.T @ Kn
            dbetan[c0:c1] += (dAn * GKnKn * EnL).sum(0)
            dgamn += (dAn * An).sum(1)
            dgamn -= (dAn * An).sum(0)
            out["dqn"][c0:c1] = np.where(resp[:, None], dQn, 0.0)
            out["dkn"][c0:c1] = np.where(resp[:, None], dKn, 0.0)
        # ---- clean: S_{c+1} = G_C S_c + K^T diag(D) U
        KdS = K @ dS
        dU += Dd[:, None] * KdS
        dD = (KdS * U).sum(1)
        dbeta[c0:c1] += dD * G[-1] / G
        dgam[-1] += (dD * Dd).sum() + G[-1] * (dS * Sc).sum()
        dgam -= dD * Dd
        dK = (Dd[:, None] * U) @ dS.T
        # o = s (diag(G) Q S_c + Mo U)
        QS = Q @ Sc
        dU += s * Mo.T @ dO
        dMo = s * dO @ U.T
        dQ = s * G[:, None] * dO @ Sc.T
        dSc += s * Q.T @ (G[:, None] * dO)
        dgam += s * G * (dO * QS).sum(1)
        # U = T rhs, rhs = V - diag(G) K S_c
        drhs = Tm.T @ dU
        dA = -drhs @ U.T
        out["dv"][c0:c1] = drhs
        dK += -G[:, None] * drhs @ Sc.T
        dSc += -K.T @ (G[:, None] * drhs)
        dgam += -G * (drhs * KS).sum(1)
        # Gram gradients, clean side
        dGo = dMo * E * bt[None, :]
        dQ += dGo @ K
        dK += dGo.T @ Q
        dbeta[c0:c1] += (dMo * GQK * E).sum(0)
        dgam += (dMo * Mo).sum(1)
        dgam -= (dMo * Mo).sum(0)
        EL = E * lower
        dGA = dA * EL * bt[None, :]
        dK += dGA @ K + dGA.T @ K
        dbeta[c0:c1] += (dA * GKK * EL).sum(0)
        dgam += (dA * A).sum(1)
        dgam -= (dA * A).sum(0)
        out["dq"][c0:c1] = dQ
        out["dk"][c0:c1] += dK
        # gamma = cumsum(log a) inside the chunk / inside each noisy block
        dga[c0:c1] = np.cumsum(dgam[::-1])[::-1]
        for s0 in range(0, L, B):
            blk = slice(s0, min(s0 + B, L))
            dgan[c0:c1][blk] = np.cumsum(dgamn[blk][::-1])[::-1]
        dS = dSc
    res = {"dq": out["dq"], "dk": out["dk"], "dv": out["dv"], "dqn": out["dqn"], "dkn": out["dkn"],
           "dvn": out["dvn"], "dalpha": dga / a, "dbeta": dbeta, "dalpha_n": np.where(np.arange(n) >= P, dgan / an, 0.0),
           "dbeta_n": np.where(np.arange(n) >= P, dbetan, 0.0), "dh0": dS}
    return res
