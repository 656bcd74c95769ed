"""fp64 numpy statement of the chunked form of KDA (TEST INFRASTRUCTURE ONLY).

The pages name the ingredients of chunked KDA (GStar Assignment 2, "Learning
path": a prefix scan of log-gates, the triangular inverse of chunked DeltaNet,
stable decayed scores) but print no formulas.  This module writes out the
rewriting of the token recurrence over a chunk of n tokens with incoming state
S, derived from the step S_t = (I - b_t k_t k_t^T) Diag(alpha_t) S_{t-1}
+ b_t k_t v_t^T, o_t = scale q_t^T S_t:

  G      = inclusive cumulative sum of log-alpha over the chunk's rows
  A_ij   = b_i sum_c K_ic K_jc exp(G_ic - G_jc)     for j < i, else 0
  P_ij   =     sum_c Q_ic K_jc exp(G_ic - G_jc)     for j <= i, else 0
  U      = (I + A)^{-1} Diag(b) (V - (K o exp(G)) S)
  O      = scale ((Q o exp(G)) S + P U)
  S_next = Diag(exp(G_last)) S + (K o exp(G_last - G))^T U

It is checked against the token recurrence of kda_oracle.c in the tests; it
exists to pin the algebra, not to be fast.  Exponent differences are formed
directly (G_ic - G_jc <= 0 for j <= i), so nothing overflows.
"""
from __future__ import annotations

import numpy as np


def chunk_step(q, k, v, la, b, S, scale=1.0):
    """One chunk: q,k [n,dk], v [n,dv], la [n,dk] log-alpha, b [n], S [dk,dv]."""
    n = k.shape[0]
    G = np.cumsum(la, axis=0)
    D = np.exp(np.minimum(G[:, None, :] - G[None, :, :], 0.0))   # [i,j,c], used for j<=i
    KK = np.einsum("ic,jc,ijc->ij", k, k, D)
    QK = np.einsum("ic,jc,ijc->ij", q, k, D) if q is not None else None
    low_strict = np.tril(np.ones((n, n)), -1)
    low_incl = np.tril(np.ones((n, n)), 0)
    A = b[:, None] * KK * low_strict
    R = b[:, None] * (v - (k * np.exp(G)) @ S)
    U = np.linalg.solve(np.eye(n) + A, R)
    out = None
    if q is not None:
        P = QK * low_incl
        out = scale * ((q * np.exp(G)) @ S + P @ U)
    g_last = G[-1]
    S_next = np.exp(g_last)[:, None] * S + (k * np.exp(g_last[None, :] - G)).T @ U
    return out, S_next


def chunked_forward(q, k, v, la, b, S0, chunk=64, scale=1.0):
    """Whole sequence in chunks of `chunk` tokens (last chunk may be partial)."""
    n = k.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    outs = []
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        o, S = chunk_step(None if q is None else q[s:e], k[s:e], v[s:e], la[s:e], b[s:e], S, scale)
        if o is not None:
            outs.append(o)
    out = np.concatenate(outs, axis=0) if outs else None
    return out, S
