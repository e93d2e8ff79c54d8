"""Pins of the chunked (WY/UT) form against the token-by-token recurrence."""
import numpy as np
import pytest
import scipy.linalg

from oracle import chunk, gdn


def _rand(rng, n, dk, dv, T, alo=0.05):
    q = rng.standard_normal((T, n, dk))
    k = rng.standard_normal((T, n, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, n, dv))
    a = rng.uniform(alo, 0.999, (T, n))
    b = rng.uniform(0.01, 0.999, (T, n))
    return q, k, v, a, b


@pytest.mark.parametrize("C", [1, 2, 4, 8, 16])
def test_chunk_equals_sequential(C):
    rng = np.random.default_rng(C)
    n, dk, dv = 5, 16, 12
    q, k, v, a, b = _rand(rng, n, dk, dv, C)
    M0 = rng.standard_normal((n, dk, dv))
    Ms, Os = gdn.run(M0, q, k, v, a, b)
    Mc, Oc = chunk.period(M0, q, k, v, a, b)
    scale = np.max(np.abs(Ms))
    assert np.max(np.abs(Mc - Ms)) <= 1e-12 * scale
    assert np.max(np.abs(Oc - Os)) <= 1e-12 * max(1.0, np.max(np.abs(Os)))


def test_chunk_64_with_strong_decay():
    # a 64-token chunk with small gates: cumulative gates fall towards 1e-30,
    # the log-space form stays finite and matches the recurrence
    rng = np.random.default_rng(64)
    n, dk, dv = 2, 8, 8
    q, k, v, a, b = _rand(rng, n, dk, dv, 64, alo=0.2)
    a[:] = np.minimum(a, 0.4)
    M0 = rng.standard_normal((n, dk, dv))
    Ms, Os = gdn.run(M0, q, k, v, a, b)
    Mc, Oc = chunk.period(M0, q, k, v, a, b)
    assert np.all(np.isfinite(Mc))
    np.testing.assert_allclose(Mc, Ms, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Oc, Os, rtol=1e-10, atol=1e-12)


def test_ut_transform_against_triangular_solve():
    rng = np.random.default_rng(11)
    n, C = 4, 8
    A = np.tril(rng.standard_normal((n, C, C)), -1) * 0.3
    beta = rng.uniform(0.1, 1, (C, n))
    T = chunk.ut_transform(A, beta)
    for i in range(n):
        L = np.eye(C) + beta[:, i][:, None] * A[i]
        ref = scipy.linalg.solve_triangular(L, np.diag(beta[:, i]), lower=True)
        np.testing.assert_allclose(T[i], ref, rtol=1e-12, atol=1e-14)


def test_gates_are_products_of_alpha():
    rng = np.random.default_rng(12)
    a = rng.uniform(0.1, 1, (6, 2))
    gamma, Gamma = chunk.gates(a)
    np.testing.assert_allclose(gamma, np.cumprod(a, axis=0).T, rtol=1e-13)
    for t in range(6):
        for s in range(6):
            ref = np.prod(a[s + 1:t + 1], axis=0) if s <= t else 0 * a[0]
            np.testing.assert_allclose(Gamma[:, t, s], ref, rtol=1e-13)
