"""Periodic rounding of a column-scaled low-bit GDN state (float64 reference).

Follows 'PACE: four-bit recurrent state by rounding less often': TL;DR point
(1) (the state is left unquantized while a short run of tokens is applied and
is rounded once when the run ends) and the flowchart 'Fewer roundings, less
compounded error' (decoded tokens are held back, then applied together once
per period in high precision, after which each column is re-encoded at 4 bits,
or 8 bits for the heads whose rounding errors last longest); also 'PACE: A New 4-Bit Recurrent State Quantization Method ...',
section 'Periodic Rounding: Reducing Error Accumulation'.

Readings where the pages are silent:

* Output of token t is read from the high-precision state after its own write,
  before the period-end encode (so period 1 means: update, read, round).
* A period is one call: decode the stored state, apply its tokens in order,
  encode.  A shorter final call is a shorter period.
* Heads carry a bit width each (4 or 8), fixed for every sequence.

Pinned by tests/test_oracle_pace.py: without quantization, periodic and
per-token runs agree exactly; period 1 equals an independently written
per-token-rounding loop; for periods 2..16 the accumulated error against an
unquantized run is below that of period 1 on seeded inputs.
"""
from __future__ import annotations

import numpy as np

from . import gdn, quant


def period(codes, scales, bits, q, k, v, alpha, beta):
    """One period from a stored state.

    codes [n, d_k, d_v] (integers), scales [n, d_v] float32, bits [n] or scalar;
    tokens q, k [C, n, d_k], v [C, n, d_v], alpha, beta [C, n] (float64 values).
    Returns (O [C, n, d_v], codes', scales', M_pre [n, d_k, d_v]) where M_pre
    is the high-precision state just before the period-end encode.
    """
    M = quant.decode(codes, scales)
    M, O = gdn.run(M, q, k, v, alpha, beta)
    c, s = quant.encode(M, bits)
    return O, c, s, M


def run(M_init, bits, q, k, v, alpha, beta, period_len, keep_states=False):
    """A whole decode run with periodic rounding.

    M_init [n, d_k, d_v] float64 is encoded first; then tokens are applied in
    periods of ``period_len`` (the last one may be shorter).  Returns
    (O [T, n, d_v], list of (codes, scales) after every period (the first
    entry is the initial encode), list of pre-encode states if keep_states).
    """
    codes, scales = quant.encode(M_init, bits)
    hist = [(codes, scales)]
    pre = []
    T = q.shape[0]
    O = np.empty((T,) + M_init.shape[:1] + M_init.shape[2:], dtype=np.float64)
    for t0 in range(0, T, period_len):
        t1 = min(T, t0 + period_len)
        O[t0:t1], codes, scales, M = period(codes, scales, bits, q[t0:t1],
                                            k[t0:t1], v[t0:t1], alpha[t0:t1],
                                            beta[t0:t1])
        hist.append((codes, scales))
        if keep_states:
            pre.append(M)
    return O, hist, pre
