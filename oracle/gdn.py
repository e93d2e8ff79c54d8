"""Gated delta-rule recurrence, token by token, in float64.

The pages describe the update only in words: in a gated DeltaNet the gate
controls how fast history is forgotten and the delta rule turns each write
into an online-learning gradient step, so every write interacts with the
state already stored ('低比特量化新突破：GGA+PW让线性注意力长文本生成更准更短',
section '为什么低比特状态量化会“越写越错”').  Written out with the state held as
M in R^{d_k x d_v} (row i = key channel, column j = value channel), the delta
step on the loss ||M^T k - v||^2 / 2 with step size beta, preceded by the
scalar gate alpha, is

    M_t = alpha_t * (M_{t-1} - beta_t * k_t (k_t^T M_{t-1})) + beta_t * k_t v_t^T
    o_t = M_t^T q_t

which is S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T for
S = M^T.  The read-out uses the state after the token's own write.

Pinned by tests/test_oracle_gdn.py: closed forms (beta = 0 is pure decay;
alpha = beta = 1 with a basis key overwrites one row exactly; one token from
zero), exact rational brute force on 3x3 states, column independence, and
agreement with the chunked form.
"""
from __future__ import annotations

import numpy as np


def step(M, q, k, v, alpha, beta):
    """One token for a batch of states.

    M [n, d_k, d_v]; q, k [n, d_k]; v [n, d_v]; alpha, beta [n].
    Returns (M_t, o_t [n, d_v]).
    """
    a = np.asarray(alpha, dtype=np.float64)[:, None, None]
    b = np.asarray(beta, dtype=np.float64)[:, None, None]
    kM = np.einsum("ni,nij->nj", k, M)                          # k^T M
    M = a * (M - b * k[:, :, None] * kM[:, None, :]) + b * k[:, :, None] * v[:, None, :]
    o = np.einsum("ni,nij->nj", q, M)                           # M^T q
    return M, o


def run(M0, q, k, v, alpha, beta):
    """Apply T tokens in order.  q, k [T, n, d_k]; v [T, n, d_v]; alpha, beta [T, n].

    Returns (M_T [n, d_k, d_v], O [T, n, d_v]).
    """
    M = np.array(M0, dtype=np.float64, copy=True)
    T = q.shape[0]
    O = np.empty((T,) + M.shape[:1] + M.shape[2:], dtype=np.float64)
    for t in range(T):
        M, O[t] = step(M, q[t], k[t], v[t], alpha[t], beta[t])
    return M, O


def from_zero(d_k, d_v, q, k, v, alpha, beta):
    """State after T unquantized tokens starting from the zero state."""
    n = q.shape[1]
    M, _ = run(np.zeros((n, d_k, d_v)), q, k, v, alpha, beta)
    return M
