"""Pins of the buffered per-step oracle (oracle/buffered.py) against the
period-call oracle (oracle/pace.py), which is written and pinned separately."""
import numpy as np
import pytest

from oracle import buffered, gdn, quant
from oracle import pace as opace


def _tokens(rng, T, n, dk, dv):
    q = rng.standard_normal((T, n, dk))
    k = rng.standard_normal((T, n, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, n, dv))
    a = rng.uniform(0.6, 1.0, (T, n))
    b = rng.uniform(0.1, 0.9, (T, n))
    return q, k, v, a, b


@pytest.mark.parametrize("period", [1, 3, 4])
def test_all_active_equals_period_calls(period):
    rng = np.random.default_rng(period)
    n, dk, dv, T = 5, 16, 12, 13                     # 13 steps: a short last period
    bits = np.array([4, 8, 4, 4, 8])
    M0 = rng.standard_normal((n, dk, dv))
    q, k, v, a, b = _tokens(rng, T, n, dk, dv)
    O, hist, _ = opace.run(M0, bits, q, k, v, a, b, period)
    c0, s0 = quant.encode(M0, bits)
    st = buffered.Buffered(c0, s0, bits, period)
    ends = 0
    for t in range(T):
        o = st.step(q[t], k[t], v[t], a[t], b[t])
        np.testing.assert_allclose(o, O[t], rtol=1e-12, atol=1e-12)
        assert np.all(st.fill == (t + 1) % period)
        if (t + 1) % period == 0:
            ends += 1
            np.testing.assert_array_equal(st.codes, hist[ends][0])
            np.testing.assert_array_equal(st.scales, hist[ends][1])
    st.flush()
    assert np.all(st.fill == 0)
    np.testing.assert_array_equal(st.codes, hist[-1][0])
    np.testing.assert_array_equal(st.scales, hist[-1][1])


def test_skipped_steps_keep_each_buffer():
    # states skipped by a step keep their buffer: each state's outputs equal a
    # period-call run over its own active tokens only
    rng = np.random.default_rng(7)
    n, dk, dv, T, period = 4, 8, 8, 20, 4
    bits = np.array([4, 8, 4, 4])
    M0 = rng.standard_normal((n, dk, dv))
    q, k, v, a, b = _tokens(rng, T, n, dk, dv)
    act = rng.uniform(size=(T, n)) < 0.6
    act[0] = True
    c0, s0 = quant.encode(M0, bits)
    st = buffered.Buffered(c0, s0, bits, period)
    outs = np.stack([st.step(q[t], k[t], v[t], a[t], b[t], act[t]) for t in range(T)])
    st.flush()
    assert len(set(st.fill.tolist())) == 1
    for i in range(n):
        ts = np.nonzero(act[:, i])[0]
        sel = [x[ts][:, i:i + 1] for x in (q, k, v, a, b)]
        O, hist, _ = opace.run(M0[i:i + 1], bits[i:i + 1], *sel, period)
        np.testing.assert_allclose(outs[ts, i], O[:, 0], rtol=1e-12, atol=1e-12)
        assert np.all(np.isnan(outs[~act[:, i], i]))
        np.testing.assert_array_equal(st.codes[i], hist[-1][0][0])
        np.testing.assert_array_equal(st.scales[i], hist[-1][1][0])


def test_period_one_rounds_every_token():
    rng = np.random.default_rng(3)
    n, dk, dv, T = 3, 8, 8, 6
    M0 = rng.standard_normal((n, dk, dv))
    q, k, v, a, b = _tokens(rng, T, n, dk, dv)
    c, s = quant.encode(M0, 4)
    st = buffered.Buffered(c, s, 4, 1)
    for t in range(T):
        o = st.step(q[t], k[t], v[t], a[t], b[t])
        M, o_ref = gdn.step(quant.decode(c, s), q[t], k[t], v[t], a[t], b[t])
        c, s = quant.encode(M, 4)
        np.testing.assert_allclose(o, o_ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(st.codes, c)
        assert np.all(st.fill == 0)


def test_buffer_never_holds_a_full_period():
    rng = np.random.default_rng(4)
    n, d, period = 2, 8, 5
    c, s = quant.encode(rng.standard_normal((n, d, d)), 4)
    st = buffered.Buffered(c, s, 4, period)
    q, k, v, a, b = _tokens(rng, 12, n, d, d)
    for t in range(12):
        st.step(q[t], k[t], v[t], a[t], b[t])
        assert st.fill.max() <= period - 1


def _adaptive_run(period, tau, T=14, seed=11):
    rng = np.random.default_rng(seed)
    n, dk, dv = 3, 8, 8
    bits = np.array([4, 8, 4])
    M0 = rng.standard_normal((n, dk, dv))
    toks = _tokens(rng, T, n, dk, dv)
    c0, s0 = quant.encode(M0, bits)
    st = buffered.Buffered(c0, s0, bits, period, tau=tau)
    outs = [st.step(*(x[t] for x in toks)) for t in range(T)]
    return M0, bits, toks, st, np.stack(outs)


def test_adaptive_never_crossing_is_the_fixed_period():
    M0, bits, toks, st, outs = _adaptive_run(period=5, tau=1e30)
    O, hist, _ = opace.run(M0, bits, *toks, 5)
    np.testing.assert_allclose(outs, O, rtol=1e-12, atol=1e-12)
    st.flush()
    np.testing.assert_array_equal(st.codes, hist[-1][0])


def test_adaptive_tiny_threshold_is_period_two():
    # any buffered write crosses tau * R: the second token of each period closes it
    M0, bits, toks, st, outs = _adaptive_run(period=6, tau=1e-30)
    O, hist, _ = opace.run(M0, bits, *toks, 2)
    np.testing.assert_allclose(outs, O, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(st.codes, hist[-1][0])
    np.testing.assert_array_equal(st.scales, hist[-1][1])


def test_update_norm_is_the_write_into_the_state():
    # A grows by ||M_t - alpha_t M_{t-1}||_F (the token's write), computed here
    # from the recurrence itself; R is the decoded stored state's norm
    rng = np.random.default_rng(2)
    n, d = 2, 8
    c, s = quant.encode(rng.standard_normal((n, d, d)), 4)
    st = buffered.Buffered(c, s, 4, 8, tau=1e30)
    np.testing.assert_allclose(st.R, np.linalg.norm(quant.decode(c, s), axis=(1, 2)))
    q, k, v, a, b = _tokens(rng, 3, n, d, d)
    M = quant.decode(c, s)
    A = np.zeros(n)
    for t in range(3):
        Mn, _ = gdn.step(M, q[t], k[t], v[t], a[t], b[t])
        A += np.linalg.norm(Mn - a[t][:, None, None] * M, axis=(1, 2))
        st.step(q[t], k[t], v[t], a[t], b[t])
        np.testing.assert_allclose(st.A, A, rtol=1e-12)
        M = Mn


def test_adaptive_threshold_between_periods():
    # a moderate threshold gives periods between 2 and the maximum, and
    # every close happens exactly when A > tau R held before the step
    rng = np.random.default_rng(9)
    n, d, kmax, tau = 4, 8, 8, 0.5
    c, s = quant.encode(rng.standard_normal((n, d, d)), 4)
    st = buffered.Buffered(c, s, 4, kmax, tau=tau)
    q, k, v, a, b = _tokens(rng, 40, n, d, d)
    lengths = []
    for t in range(40):
        fill = st.fill.copy()
        expect = [(fill[i] + 1 == kmax) or (st.A[i] > tau * st.R[i]) for i in range(n)]
        st.step(q[t], k[t], v[t], a[t], b[t])
        for i in range(n):
            assert (st.fill[i] == 0) == expect[i]
            if expect[i]:
                lengths.append(fill[i] + 1)
    assert 2 <= min(lengths) and max(lengths) <= kmax and len(set(lengths)) > 1
