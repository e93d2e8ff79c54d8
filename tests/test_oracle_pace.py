"""Pins of periodic rounding in the oracle (oracle/pace.py).

The pages claim two things checkable without trained weights: rounding once
per period instead of once per token accumulates less error, and per-column
scales fit gated-delta states whose large entries sit in columns.  Both are
checked here on seeded synthetic inputs, together with the exact reductions
(no quantization; period 1 = per-token rounding).
"""
import numpy as np
import pytest

from linear_attn_decode_pace_amd import inputs
from oracle import gdn, pace, quant


def _tiles(tok, name):
    a = tok.f64(name)
    return a.reshape((a.shape[0], -1) + a.shape[3:])


def _toks(w, seed, t0, t1, seg=inputs.SEG_DECODE):
    tok = inputs.tokens(w, seed, seg, t0, t1)
    return [_tiles(tok, n) for n in ("q", "k", "v", "alpha", "beta")]


def _warm(w, seed):
    q, k, v, a, b = _toks(w, seed, 0, w.warmup, inputs.SEG_WARMUP)
    return gdn.from_zero(w.dk, w.dv, q, k, v, a, b)


def test_unquantized_periodic_equals_per_token():
    w = inputs.TINY.replace(B=2, dk=16, dv=16)
    q, k, v, a, b = _toks(w, 0, 0, 24)
    M0 = _warm(w, 0)
    M1, O1 = gdn.run(M0, q, k, v, a, b)
    M = M0
    O = []
    for t0 in range(0, 24, 8):          # periods of 8 without any rounding
        M, o = gdn.run(M, q[t0:t0 + 8], k[t0:t0 + 8], v[t0:t0 + 8], a[t0:t0 + 8], b[t0:t0 + 8])
        O.append(o)
    assert np.array_equal(M, M1)
    assert np.array_equal(np.concatenate(O), O1)


def _per_token_rounding_loop(M0, bits, q, k, v, a, b):
    """Independent per-token rounding: plain loops over tiles and columns."""
    qm = 2 ** (bits - 1) - 1
    n, dk, dv = M0.shape

    def enc(M):
        C = np.zeros_like(M)
        S = np.zeros((n, dv), dtype=np.float32)
        for i in range(n):
            for j in range(dv):
                amax = max(abs(x) for x in M[i, :, j])
                s = np.float32(amax / qm)
                S[i, j] = s
                if s > 0:
                    for r in range(dk):
                        C[i, r, j] = min(qm, max(-qm, np.rint(M[i, r, j] / float(s))))
        return C, S

    C, S = enc(M0)
    outs = []
    for t in range(q.shape[0]):
        M = C * S.astype(np.float64)[:, None, :]
        for i in range(n):
            kM = k[t, i] @ M[i]
            M[i] = a[t, i] * (M[i] - b[t, i] * np.outer(k[t, i], kM)) + b[t, i] * np.outer(k[t, i], v[t, i])
        outs.append(np.einsum("ni,nij->nj", q[t], M))
        C, S = enc(M)
    return np.array(outs), C, S


@pytest.mark.parametrize("bits", [4, 8])
def test_period_one_is_per_token_rounding(bits):
    w = inputs.TINY.replace(B=2, H=1, dk=8, dv=6, warmup=8)
    q, k, v, a, b = _toks(w, 1, 0, 6)
    M0 = _warm(w, 1)
    O, hist, _ = pace.run(M0, bits, q, k, v, a, b, 1)
    Oref, Cref, Sref = _per_token_rounding_loop(M0, bits, q, k, v, a, b)
    np.testing.assert_allclose(O, Oref, rtol=1e-12, atol=1e-14)
    assert np.array_equal(hist[-1][0], Cref.astype(np.int16))
    assert np.array_equal(hist[-1][1], Sref)


def test_period_outputs_are_read_before_the_encode():
    w = inputs.TINY.replace(B=1, H=2, dk=16, dv=16)
    q, k, v, a, b = _toks(w, 2, 0, 4)
    M0 = _warm(w, 2)
    c, s = quant.encode(M0, 4)
    O, c2, s2, Mpre = pace.period(c, s, 4, q, k, v, a, b)
    Mref, Oref = gdn.run(quant.decode(c, s), q, k, v, a, b)
    assert np.array_equal(O, Oref) and np.array_equal(Mpre, Mref)
    c3, s3 = quant.encode(Mref, 4)
    assert np.array_equal(c2, c3) and np.array_equal(s2, s3)


def _rel(x, ref):
    return np.linalg.norm(x - ref) / np.linalg.norm(ref)


def test_fewer_roundings_accumulate_less_error():
    # 'PACE: four-bit recurrent state by rounding less often', TL;DR (1):
    # rounding once per period compounds less error than once per token.
    w = inputs.SWEEP.replace(B=4, H=6, dk=64, dv=64, dtype=inputs.DT_F32)
    T = 128
    q, k, v, a, b = _toks(w, 3, 0, T)
    M0 = _warm(w, 3)
    Mx, Ox = gdn.run(M0, q, k, v, a, b)
    err = {}
    for per in (1, 2, 4, 8, 16):
        O, hist, _ = pace.run(M0, 4, q, k, v, a, b, per)
        err[per] = _rel(O, Ox)
    for per in (2, 4, 8, 16):
        assert err[per] < err[1], err
    assert err[16] < err[4] < err[1], err


def test_column_scales_beat_row_scales_with_column_outliers():
    # 'PACE: A New 4-Bit ...', section 'Channel-Aligned Encoding': large
    # entries cluster in columns, so one scale per column fits them better.
    w = inputs.MIXED.replace(B=4, H=4, dk=64, dv=64, n_int8=0)
    M = _warm(w, 4)
    c, s = quant.encode(M, 4)
    e_col = _rel(quant.decode(c, s), M)
    Mt = np.transpose(M, (0, 2, 1))          # same quantizer, one scale per key row
    cr, sr = quant.encode(Mt, 4)
    e_row = _rel(np.transpose(quant.decode(cr, sr), (0, 2, 1)), M)
    assert e_col < 0.8 * e_row, (e_col, e_row)
