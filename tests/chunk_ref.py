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
