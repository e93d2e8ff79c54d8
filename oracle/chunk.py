"""Chunked (WY / UT) form of one period of the gated delta rule, float64.

Used only to pin that applying a period's tokens as one chunk gives the same
state and outputs as the token-by-token recurrence; the pages name chunked
kernels as the origin of periodic rounding ('PACE: four-bit recurrent state by
rounding less often', TL;DR point (1); 'PACE: A New 4-Bit Recurrent State
Quantization Method ...', section 'Periodic Rounding': chunks are computed in
parallel inside and pass state between them).  The algebra is derived from
the recurrence in ``gdn``: unrolling it over C tokens gives

    M_t = gamma_t M_0 + sum_{s<=t} Gamma_ts k_s u_s^T
    gamma_t = prod_{r<=t} alpha_r,  Gamma_ts = prod_{s<r<=t} alpha_r
    u_t = beta_t (v_t - gamma_t M_0^T k_t - sum_{s<t} Gamma_ts (k_t.k_s) u_s)

so with tokens as rows (K, Q [C, d_k], V, U, O [C, d_v]):

    A   = strictly lower part of (Gamma * K K^T)
    T   = (I + diag(beta) A)^-1 diag(beta)        (forward substitution)
    U   = T (V - diag(gamma) K M_0)
    O   = diag(gamma) Q M_0 + lower part incl. diagonal of (Gamma * Q K^T) U
    M_C = gamma_C M_0 + K^T diag(Gamma_C,:) U

Pinned by tests/test_oracle_chunk.py against ``gdn.run`` and, for T, against
scipy.linalg.solve_triangular.
"""
from __future__ import annotations

import numpy as np


def gates(alpha):
    """alpha [C, n] -> (gamma [n, C], Gamma [n, C, C]) from cumulative log gates."""
    g = np.cumsum(np.log(np.asarray(alpha, dtype=np.float64)), axis=0).T   # [n, C]
    gamma = np.exp(g)
    diff = g[:, :, None] - g[:, None, :]
    C = g.shape[1]
    low = np.tril(np.ones((C, C), dtype=bool))
    Gamma = np.where(low, np.exp(np.where(low, diff, 0.0)), 0.0)
    return gamma, Gamma


def ut_transform(A, beta):
    """T = (I + diag(beta) A)^-1 diag(beta) for strictly lower A [n, C, C],
    by forward substitution, row by row."""
    n, C, _ = A.shape
    b = np.asarray(beta, dtype=np.float64).T                # [n, C]
    Z = np.zeros((n, C, C))
    for t in range(C):
        row = np.zeros((n, C))
        row[:, t] = 1.0
        for s in range(t):
            row -= (b[:, t] * A[:, t, s])[:, None] * Z[:, s, :]
        Z[:, t, :] = row
    return Z * b[:, None, :]


def period(M0, q, k, v, alpha, beta):
    """One chunk.  M0 [n, d_k, d_v]; q, k [C, n, d_k]; v [C, n, d_v]; alpha, beta [C, n].
    Returns (M_C, O [C, n, d_v])."""
    K = np.transpose(k, (1, 0, 2))
    Q = np.transpose(q, (1, 0, 2))
    V = np.transpose(v, (1, 0, 2))
    gamma, Gamma = gates(alpha)
    C = K.shape[1]
    A = np.tril(Gamma * (K @ np.transpose(K, (0, 2, 1))), -1)
    T = ut_transform(A, beta)
    U = T @ (V - gamma[:, :, None] * (K @ M0))
    P = np.tril(Gamma * (Q @ np.transpose(K, (0, 2, 1))))
    O = gamma[:, :, None] * (Q @ M0) + P @ U
    W = Gamma[:, C - 1, :, None] * U
    M = gamma[:, C - 1, None, None] * M0 + np.transpose(K, (0, 2, 1)) @ W
    return M, np.transpose(O, (1, 0, 2))
