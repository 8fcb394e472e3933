"""fp64 chunked (WY / UT) form of the KDA recurrence, test-only.

Derived from the token loop by unrolling one chunk of C tokens from its entry
state S0, with G_i = sum_{s<=i} log_g_s (per key channel, inclusive) and
gamma = G_{C-1}:

    A[i,j]   = beta_i sum_c k_ic k_jc exp(G_ic - G_jc)      (j < i)
    (I + A) Delta = beta*V - (beta*K*exp(G)) S0
    Aqk[i,j] = sum_c q_ic k_jc exp(G_ic - G_jc)             (j <= i)
    O        = scale ((Q*exp(G)) S0 + Aqk Delta)
    S_next   = exp(gamma) * S0 + (K*exp(gamma - G))^T Delta

This is the algebra the GPU prefill kernel evaluates; the tests check it against
the oracle's token loop for several chunk sizes.  Pairwise exponents are formed
as differences (never exp(G) * exp(-G)) so that strong decays stay finite.
"""
import numpy as np


def chunk_forward(q, k, v, log_g, beta, S0, scale, C):
    """One unit: q, k, log_g [T, dk]; v [T, dv]; beta [T]; S0 [dk, dv]."""
    T, dk = q.shape
    dv = v.shape[1]
    S = np.array(S0, dtype=np.float64, copy=True)
    out = np.zeros((T, dv))
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        n = sl.stop - sl.start
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        G = np.cumsum(log_g[sl], axis=0)
        gam = G[-1]
        D = G[:, None, :] - G[None, :, :]            # [i, j, c] = G_ic - G_jc
        tri = np.tril(np.ones((n, n), dtype=bool))
        E = np.where(tri[:, :, None], np.exp(np.where(tri[:, :, None], D, 0.0)), 0.0)
        Akk = np.einsum('ic,jc,ijc->ij', K, K, E)
        A = b[:, None] * np.tril(Akk, -1)
        Aqk = np.einsum('ic,jc,ijc->ij', Q, K, E)
        rhs = b[:, None] * V - (b[:, None] * K * np.exp(G)) @ S
        Delta = np.linalg.solve(np.eye(n) + A, rhs)
        out[sl] = scale * ((Q * np.exp(G)) @ S + Aqk @ Delta)
        S = np.exp(gam)[:, None] * S + (K * np.exp(gam[None, :] - G)).T @ Delta
    return out, S


def _pair(X, Y, E):
    """M[t, s] = sum_c X[t, c] Y[s, c] E[t, s, c]."""
    return np.einsum('tc,sc,tsc->ts', X, Y, E)


def _pair_grads(dM, X, Y, E):
    """Gradients of M = _pair(X, Y, E) with E[t, s, c] = exp(G_tc - G_sc):
    (dX, dY, dG), where G enters with + through t and - through s."""
    W = dM[:, :, None] * E                       # [t, s, c]
    dX = np.einsum('tsc,sc->tc', W, Y)
    dY = np.einsum('tsc,tc->sc', W, X)
    dG = X * dX - Y * dY
    return dX, dY, dG


def chunk_backward(q, k, v, log_g, beta, S0, scale, C, d_out, d_final):
    """Reverse mode of chunk_forward for one unit, in chunk form.

    Per chunk, with S the entry state and dS the gradient of the exit state
    (the backward pass of the chunk algebra above, term by term):

        dDelta = scale Aqk^T dO + Kd dS
        dR     = (I + A)^-T dDelta                 R = beta (V - Kb S)
        dA     = -tril(dR Delta^T, -1),  dAqk = scale tril(dO Delta^T)
        dbeta  = rowsum(dR * (V - Kb S)) + rowsum(dA * Akk)
        dV     = beta dR,  dKb = -beta dR S^T,  dQb = scale dO S^T,  dKd = Delta dS^T
        dS_in  = exp(gamma) dS + scale Qb^T dO - Kb^T (beta dR)

    and the decay-weighted pair terms pass gradients to q, k and the cumulative
    gates G, which reach log_g by a reverse cumulative sum within the chunk.
    Returns (dq, dk, dv, dlog_g, dbeta, dS0).
    """
    T, dk = q.shape
    dv = v.shape[1]
    starts = list(range(0, T, C))
    states = []
    S = np.array(S0, dtype=np.float64, copy=True)
    for c0 in starts:                             # forward: entry state of every chunk
        states.append(S.copy())
        _, S = chunk_forward(q[c0:c0 + C], k[c0:c0 + C], v[c0:c0 + C], log_g[c0:c0 + C], beta[c0:c0 + C],
                             S, scale, C)
    dq, dkk, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dlg, db = np.zeros_like(log_g), np.zeros_like(beta)
    dS = np.array(d_final, dtype=np.float64, copy=True)
    for c0, S in reversed(list(zip(starts, states))):
        sl = slice(c0, min(T, c0 + C))
        n = sl.stop - sl.start
        Q, K, V, b, dO = q[sl], k[sl], v[sl], beta[sl], d_out[sl]
        G = np.cumsum(log_g[sl], axis=0)
        gam = G[-1]
        D = G[:, None, :] - G[None, :, :]
        lower = np.tril(np.ones((n, n), dtype=bool))
        E = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], D, 0.0)), 0.0)
        Es = E * (~np.eye(n, dtype=bool))[:, :, None]    # strictly lower
        Akk = _pair(K, K, Es)
        A = b[:, None] * Akk
        Aqk = _pair(Q, K, E)
        Kb, Qb, Kd = K * np.exp(G), Q * np.exp(G), K * np.exp(gam[None, :] - G)
        Tm = np.linalg.inv(np.eye(n) + A)
        Vr = V - Kb @ S
        Delta = Tm @ (b[:, None] * Vr)
        dDelta = scale * Aqk.T @ dO + Kd @ dS
        dR = Tm.T @ dDelta
        dA = -np.tril(dR @ Delta.T, -1)
        dAqk = scale * np.tril(dO @ Delta.T)
        db[sl] = np.sum(dR * Vr, axis=1) + np.sum(dA * Akk, axis=1)
        dvv[sl] = b[:, None] * dR
        dKb = -(b[:, None] * dR) @ S.T
        dQb = scale * dO @ S.T
        dKd = Delta @ dS.T
        dG = dQb * Qb + dKb * Kb - dKd * Kd
        dgam = np.sum(dKd * Kd, axis=0) + np.exp(gam) * np.sum(dS * S, axis=1)
        x1, y1, g1 = _pair_grads(dAqk, Q, K, E)
        x2, y2, g2 = _pair_grads(b[:, None] * dA, K, K, Es)
        dq[sl] = dQb * np.exp(G) + x1
        dkk[sl] = dKb * np.exp(G) + dKd * np.exp(gam[None, :] - G) + y1 + x2 + y2
        dG = dG + g1 + g2
        dG[-1] += dgam
        dlg[sl] = np.cumsum(dG[::-1], axis=0)[::-1]
        dS = np.exp(gam)[:, None] * dS + scale * Qb.T @ dO - Kb.T @ (b[:, None] * dR)
    return dq, dkk, dvv, dlg, db, dS
