"""Exact rational brute force of the KDA recurrence in product form (test-only).

Independent of the oracle's token loop: the state after t tokens is written as
a product of per-token transition matrices,

    S_t = P_t ... P_1 S_0 + sum_{s<=t} P_t ... P_{s+1} (beta_s k_s v_s^T),
    P_s = (I - beta_s k_s k_s^T) Diag(alpha_s),

which follows from the gated delta rule of the GLM-5.3-Flash model notes
(Glm5NextTextLinearAttention snippet): decaying the key axis is Diag(alpha) S,
and the update S' + k beta (v - S'^T k)^T equals (I - beta k k^T) S' + beta k v^T.
Outputs o_t = scale S_t^T q_t.  Everything is fractions.Fraction.
"""
from fractions import Fraction


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][l] * B[l][j] for l in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def _add(A, B):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


def _eye(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def transition(alpha, beta, k):
    dk = len(k)
    D = [[alpha[i] if i == j else Fraction(0) for j in range(dk)] for i in range(dk)]
    M = [[Fraction(int(i == j)) - beta * k[i] * k[j] for j in range(dk)] for i in range(dk)]
    return _matmul(M, D)


def run(alpha, beta, k, v, q, S0, scale):
    """alpha, k, q: [T][dk]; v: [T][dv]; beta: [T]; S0: [dk][dv] (Fractions).

    Returns (outputs [T][dv], S_T [dk][dv]) built from prefix products of the
    transition matrices (no token-loop update of a running state)."""
    T, dk, dv = len(alpha), len(S0), len(S0[0])
    P = [transition(alpha[s], beta[s], k[s]) for s in range(T)]
    inj = [[[beta[s] * k[s][i] * v[s][j] for j in range(dv)] for i in range(dk)] for s in range(T)]
    outs, S_t = [], None
    for t in range(T):
        # S_t = (P_t...P_0) S0 + sum_{s<=t} (P_t...P_{s+1}) inj_s
        prod = _eye(dk)
        S_t = [[Fraction(0)] * dv for _ in range(dk)]
        for s in range(t, -1, -1):
            S_t = _add(S_t, _matmul(prod, inj[s]))
            prod = _matmul(prod, P[s])
        S_t = _add(S_t, _matmul(prod, S0))
        outs.append([scale * sum((S_t[i][j] * q[t][i] for i in range(dk)), Fraction(0))
                     for j in range(dv)])
    return outs, S_t if S_t is not None else [row[:] for row in S0]
