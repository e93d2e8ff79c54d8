"""Pins of the oracle's gated delta-rule recurrence (oracle/gdn.py).

Each check is fixed by mathematics, not by the oracle: closed forms, an exact
rational brute force written here independently, and structural invariants.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import gdn


def _rand(rng, n, dk, dv, T):
    q = rng.standard_normal((T, n, dk))
    k = rng.standard_normal((T, n, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, n, dv))
    a = rng.uniform(0.05, 0.99, (T, n))
    b = rng.uniform(0.05, 0.99, (T, n))
    return q, k, v, a, b


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(1)
    n, dk, dv, T = 3, 6, 5, 7
    q, k, v, a, _ = _rand(rng, n, dk, dv, T)
    M0 = rng.standard_normal((n, dk, dv))
    M, O = gdn.run(M0, q, k, v, a, np.zeros((T, n)))
    gamma = np.cumprod(a, axis=0)
    np.testing.assert_allclose(M, gamma[-1][:, None, None] * M0, rtol=1e-13)
    for t in range(T):
        ref = gamma[t][:, None] * np.einsum("ni,nij->nj", q[t], M0)
        np.testing.assert_allclose(O[t], ref, rtol=1e-12, atol=1e-14)


def test_basis_key_overwrites_one_row_exactly():
    rng = np.random.default_rng(2)
    dk, dv = 5, 4
    M0 = rng.standard_normal((1, dk, dv))
    for i in range(dk):
        k = np.zeros((1, 1, dk))
        k[0, 0, i] = 1.0
        v = rng.standard_normal((1, 1, dv))
        q = rng.standard_normal((1, 1, dk))
        M, _ = gdn.run(M0, q, k, v, np.ones((1, 1)), np.ones((1, 1)))
        expect = M0.copy()
        expect[0, i, :] = v[0, 0]
        assert np.array_equal(M, expect)


def test_one_token_from_zero():
    rng = np.random.default_rng(3)
    n, dk, dv = 4, 8, 6
    q, k, v, a, b = _rand(rng, n, dk, dv, 1)
    M, O = gdn.run(np.zeros((n, dk, dv)), q, k, v, a, b)
    ref = b[0][:, None, None] * k[0][:, :, None] * v[0][:, None, :]
    np.testing.assert_allclose(M, ref, rtol=1e-15, atol=0)
    # the output reads the state after the token's own write: beta (k.q) v
    ref_o = (b[0] * np.sum(k[0] * q[0], axis=-1))[:, None] * v[0]
    np.testing.assert_allclose(O[0], ref_o, rtol=1e-14, atol=1e-16)


def test_delta_rule_maps_key_to_value():
    # With alpha = beta = 1 and a unit key the write makes the state return the
    # written value for that key: M_t^T k_t = v_t (the delta rule's fixed point).
    rng = np.random.default_rng(4)
    n, dk, dv = 5, 16, 16
    q, k, v, _, _ = _rand(rng, n, dk, dv, 1)
    M0 = rng.standard_normal((n, dk, dv))
    M, _ = gdn.run(M0, q, k, v, np.ones((1, n)), np.ones((1, n)))
    np.testing.assert_allclose(np.einsum("ni,nij->nj", k[0], M), v[0],
                               rtol=1e-12, atol=1e-12)


def _exact_run(M0, q, k, v, a, b):
    """Token-by-token recurrence in exact rational arithmetic (pure Python)."""
    dk, dv = len(M0), len(M0[0])
    M = [[Fraction(x) for x in row] for row in M0]
    outs = []
    for t in range(len(q)):
        kM = [sum(Fraction(k[t][i]) * M[i][j] for i in range(dk)) for j in range(dv)]
        A, B = Fraction(a[t]), Fraction(b[t])
        M = [[A * (M[i][j] - B * Fraction(k[t][i]) * kM[j]) + B * Fraction(k[t][i]) * Fraction(v[t][j])
              for j in range(dv)] for i in range(dk)]
        outs.append([sum(Fraction(q[t][i]) * M[i][j] for i in range(dk)) for j in range(dv)])
    return M, outs


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_exact_rational_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    dk = dv = 3
    T = 4
    # inputs are binary fractions, so float64 holds them exactly
    q = np.round(rng.uniform(-1, 1, (T, dk)) * 64) / 64
    k = np.round(rng.uniform(-1, 1, (T, dk)) * 64) / 64
    v = np.round(rng.uniform(-2, 2, (T, dv)) * 64) / 64
    a = np.round(rng.uniform(0.1, 1, T) * 256) / 256
    b = np.round(rng.uniform(0.1, 1, T) * 256) / 256
    M0 = np.round(rng.uniform(-1, 1, (dk, dv)) * 128) / 128
    Me, Oe = _exact_run(M0.tolist(), q.tolist(), k.tolist(), v.tolist(), a.tolist(), b.tolist())
    M, O = gdn.run(M0[None], q[:, None], k[:, None], v[:, None], a[:, None], b[:, None])
    Me = np.array([[float(x) for x in row] for row in Me])
    Oe = np.array([[float(x) for x in row] for row in Oe])
    np.testing.assert_allclose(M[0], Me, rtol=0, atol=1e-14)
    np.testing.assert_allclose(O[:, 0], Oe, rtol=0, atol=1e-14)


def test_columns_are_independent():
    rng = np.random.default_rng(5)
    n, dk, dv, T = 2, 8, 6, 5
    q, k, v, a, b = _rand(rng, n, dk, dv, T)
    M0 = rng.standard_normal((n, dk, dv))
    M, O = gdn.run(M0, q, k, v, a, b)
    for j in range(dv):
        Mj, Oj = gdn.run(M0[:, :, j:j + 1], q, k, v[:, :, j:j + 1], a, b)
        np.testing.assert_allclose(Mj[:, :, 0], M[:, :, j], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(Oj[:, :, 0], O[:, :, j], rtol=1e-14, atol=1e-15)


def test_from_zero_matches_run():
    rng = np.random.default_rng(6)
    n, dk, dv, T = 3, 4, 4, 6
    q, k, v, a, b = _rand(rng, n, dk, dv, T)
    M = gdn.from_zero(dk, dv, q, k, v, a, b)
    M2, _ = gdn.run(np.zeros((n, dk, dv)), q, k, v, a, b)
    assert np.array_equal(M, M2)
