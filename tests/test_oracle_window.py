"""Pins of the FP8 write-window oracle (oracle/window.py)."""
import numpy as np
import pytest
import torch

from oracle import gdn, quant, window


def test_e4m3_decode_matches_torch_for_every_finite_code():
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]
    ref = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).float().tolist()
    assert [window.e4m3_decode_value(c) for c in codes] == ref
    assert window.e4m3_decode_value(0x7E) == 448.0


def test_e4m3_encode_matches_torch_including_ties():
    rng = np.random.default_rng(0)
    vals = list(rng.uniform(-448, 448, 2000).astype(np.float32))
    vals += list((rng.standard_normal(2000) * 2.0 ** rng.integers(-12, 4, 2000)).astype(np.float32))
    # exact midpoints between neighbouring codes (normal and subnormal) go to even
    finite = sorted({window.e4m3_decode_value(c) for c in range(0x7F)})
    vals += [np.float32((a + b) / 2) for a, b in zip(finite, finite[1:])]
    vals = [v for v in vals if abs(v) <= 448]
    ref = torch.tensor(np.array(vals, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).tolist()
    got = [window.e4m3_encode_value(float(v)) & 0xFF for v in vals]
    # torch keeps the sign of a value rounding to zero; compare magnitudes there
    for v, g, r in zip(vals, got, ref):
        assert g == r or (g & 0x7F) == (r & 0x7F) == 0, (v, g, r)


def test_fp8_vector_scale_and_range():
    x = np.array([3.0, -1.5, 0.25, 0.0])
    c, s = window.fp8_vector(x)
    assert s == np.float32(3.0) / np.float32(448.0)
    assert c[0] == 0x7E and window.e4m3_decode_value(int(c[0])) == 448.0
    np.testing.assert_allclose(window.fp8_decode(c, s), x, rtol=2 ** -4)
    z, sz = window.fp8_vector(np.zeros(5))
    assert sz == 0 and not z.any()


def _exact_tokens(T, d, rng):
    # keys 0.875 e_i on distinct rows (scale 0.875 / 448 = 2^-9); values whose
    # writes u = v / 2 have absmax 3.5 (scale 2^-7) and entries exact in E4M3
    q = rng.standard_normal((T, 1, d))
    k = np.zeros((T, 1, d))
    k[np.arange(T), 0, rng.permutation(d)[:T]] = 0.875
    v = rng.choice([-6.0, -4.0, -3.5, -2.0, -1.75, 1.0, 2.0, 3.5, 4.0, 6.0], size=(T, 1, d))
    v[:, 0, 0] = 7.0
    a = rng.choice([0.5, 0.75, 1.0], size=(T, 1))
    b = np.full((T, 1), 0.5)
    return q, k, v, a, b


def test_window_without_merges_is_the_exact_recurrence():
    # keys on distinct rows from a zero state: every write u_t = beta v_t is
    # exact in FP8, so the windowed state is the recurrence itself
    rng = np.random.default_rng(1)
    T, d = 6, 16
    q, k, v, a, b = _exact_tokens(T, d, rng)
    st = window.Window(np.zeros((1, d, d)), np.zeros((1, d)), 4, S=8)
    _, O = gdn.run(np.zeros((1, d, d)), q, k, v, a, b)
    for t in range(T):
        # equal up to float64 summation order
        np.testing.assert_allclose(st.step(q[t], k[t], v[t], a[t], b[t]), O[t], rtol=1e-13, atol=1e-13)
    assert not st.codes.any()       # nothing merged: the history is still zero


def test_merge_rounds_the_oldest_write_into_the_history():
    # S = 2: from the third token on, each step merges the write made two
    # steps earlier; check the history against encode(lam H + delta k u^T)
    rng = np.random.default_rng(2)
    d, T = 8, 6
    c0, s0 = quant.encode(rng.standard_normal((1, d, d)), 8)
    st = window.Window(c0, s0, 8, S=2)
    q = rng.standard_normal((T, 1, d))
    k = rng.standard_normal((T, 1, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, 1, d))
    a = rng.uniform(0.6, 1.0, (T, 1))
    b = rng.uniform(0.2, 0.8, (T, 1))
    for t in range(T):
        before = [list(e) for e in st.win[0]]
        lam, c, s = st.lam[0], st.codes[0].copy(), st.scales[0].copy()
        st.step(q[t], k[t], v[t], a[t], b[t])
        if t >= 2:
            kc, ks, uc, us, delta = before[0]
            H = lam * a[t, 0] * quant.decode(c, s) + \
                delta * a[t, 0] * np.outer(window.fp8_decode(kc, ks), window.fp8_decode(uc, us))
            rc, rs = quant.encode(H[None], 8)
            np.testing.assert_array_equal(st.codes[0], rc[0])
            assert st.lam[0] == 1.0 and len(st.win[0]) == 2
        else:
            assert len(st.win[0]) == t + 1


def test_window_tracks_the_recurrence_closely():
    # with real data the only differences are FP8 and the history's rounding:
    # outputs stay within a few percent of the unquantized recurrence
    rng = np.random.default_rng(3)
    n, d, T = 3, 16, 24
    M0 = rng.standard_normal((n, d, d))
    c0, s0 = quant.encode(M0, 8)
    q = rng.standard_normal((T, n, d))
    k = rng.standard_normal((T, n, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, n, d))
    a = rng.uniform(0.8, 1.0, (T, n))
    b = rng.uniform(0.2, 0.8, (T, n))
    st = window.Window(c0, s0, 8, S=8)
    _, O = gdn.run(quant.decode(c0, s0), q, k, v, a, b)
    out = np.stack([st.step(q[t], k[t], v[t], a[t], b[t]) for t in range(T)])
    rel = np.linalg.norm(out - O) / np.linalg.norm(O)
    assert rel < 0.05, rel
    st.flush()
    assert all(len(w) == 0 for w in st.win) and np.all(st.lam == 1.0)


def _flush_case(seed, T=5, d=16, S=8):
    """A history on rows 0..d/2-1 (exactly representable codes) and T writes
    on distinct rows of the other half: each key row of the state is still
    zero when its token arrives, so every write is u_t = beta v_t, exact in
    E4M3, and all float64 sums below are exact (dyadic gates)."""
    rng = np.random.default_rng(seed)
    H0 = rng.standard_normal((1, d, d))
    H0[:, d // 2:, :] = 0
    c0, s0 = quant.encode(H0, 8)
    q = rng.standard_normal((T, 1, d))
    k = np.zeros((T, 1, d))
    k[np.arange(T), 0, d // 2 + rng.permutation(d // 2)[:T]] = 0.875
    v = rng.choice([-6.0, -4.0, -3.5, -2.0, -1.75, 1.0, 2.0, 3.5, 4.0, 6.0], size=(T, 1, d))
    v[:, 0, 0] = 7.0
    a = rng.choice([0.5, 0.75], size=(T, 1))    # every gate decays history and writes
    b = np.full((T, 1), 0.5)
    return c0, s0, q, k, v, a, b, S


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_flush_equals_encode_of_the_recurrence(seed):
    # a flush with no merge before it must store encode(M_T) of the plain
    # recurrence: the history decayed by every gate (lam), each write decayed
    # by the gates after it (delta), all in one encode
    c0, s0, q, k, v, a, b, S = _flush_case(seed)
    T = q.shape[0]
    st = window.Window(c0, s0, 8, S=S)
    for t in range(T):
        st.step(q[t], k[t], v[t], a[t], b[t])
    # no write has left the window yet: the stored history is untouched
    assert len(st.win[0]) == T and np.array_equal(st.codes[0], c0[0])
    MT, _ = gdn.run(quant.decode(c0, s0), q, k, v, a, b)
    st.flush()
    rc, rs = quant.encode(MT, 8)
    np.testing.assert_array_equal(st.last_pre[0], MT[0])      # exact sums
    np.testing.assert_array_equal(st.codes[0], rc[0])
    np.testing.assert_array_equal(st.scales[0], rs[0])
    assert st.lam[0] == 1.0 and st.win[0] == []


@pytest.mark.parametrize("seed", [3, 4])
def test_flush_encodes_the_state_it_holds(seed):
    # with real data (and merges before it), a flush encodes exactly the state
    # that state() reports just before it
    rng = np.random.default_rng(seed)
    n, d, T, S = 3, 16, 11, 4
    c0, s0 = quant.encode(rng.standard_normal((n, d, d)), np.array([4, 8, 4]))
    st = window.Window(c0, s0, np.array([4, 8, 4]), S=S)
    q = rng.standard_normal((T, n, d))
    k = rng.standard_normal((T, n, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, n, d))
    a = rng.uniform(0.5, 1.0, (T, n))
    b = rng.uniform(0.2, 0.8, (T, n))
    for t in range(T):
        st.step(q[t], k[t], v[t], a[t], b[t])
    before = [st.state(i) for i in range(n)]
    st.flush()
    for i in range(n):
        np.testing.assert_allclose(st.last_pre[i], before[i], rtol=1e-14, atol=1e-15)
        rc, rs = quant.encode(before[i][None], st.bits[i:i + 1])
        np.testing.assert_array_equal(st.codes[i], rc[0])
        np.testing.assert_array_equal(st.scales[i], rs[0])
