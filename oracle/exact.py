"""Exact-rational KDA recurrence and affine scan (TEST INFRASTRUCTURE ONLY).

A second, independent statement of the token step in fractions.Fraction
arithmetic, for tiny inputs whose alpha and beta are supplied directly as
rationals.  The step follows the nx_nofloat_kda.nx source (header comment,
kda_gate then kda_write then the read-out): decay each key row by its channel
gate, predict from the decayed state, delta-write, read the updated state.
The scan follows KDA Context Parallelism, "Implementation order".
"""
from __future__ import annotations

from fractions import Fraction as F


def _zeros(r, c):
    return [[F(0)] * c for _ in range(r)]


def exact_forward(q, k, v, alpha, beta, S0, scale=F(1)):
    """q,k: [n][dk]; v: [n][dv]; alpha: [n][dk]; beta: [n]; S0: [dk][dv].
    Returns (out [n][dv], S [dk][dv]) as Fractions."""
    S = [[F(x) for x in row] for row in S0]
    dk, dv = len(S), len(S[0])
    outs = []
    for t in range(len(k)):
        for i in range(dk):                       # decay along the key axis
            a = F(alpha[t][i])
            S[i] = [a * x for x in S[i]]
        pred = [sum(F(k[t][i]) * S[i][j] for i in range(dk)) for j in range(dv)]
        delta = [F(beta[t]) * (F(v[t][j]) - pred[j]) for j in range(dv)]
        for i in range(dk):                       # S += k delta^T
            ki = F(k[t][i])
            S[i] = [S[i][j] + ki * delta[j] for j in range(dv)]
        if q is not None:
            outs.append([F(scale) * sum(F(q[t][i]) * S[i][j] for i in range(dk))
                         for j in range(dv)])
    return outs, S


def exact_matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum(A[i][c] * B[c][j] for c in range(m)) for j in range(p)] for i in range(n)]


def exact_scan(Ms, Us, S_init):
    """Exclusive prefix of affine maps, in segment order, exact."""
    W = [[F(x) for x in row] for row in S_init]
    inc, outg = [], []
    for M, U in zip(Ms, Us):
        inc.append(W)
        MW = exact_matmul([[F(x) for x in r] for r in M], W)
        W = [[MW[i][j] + F(U[i][j]) for j in range(len(W[0]))] for i in range(len(W))]
        outg.append(W)
    return {"incoming_states": inc, "outgoing_states": outg, "final_state": W}
