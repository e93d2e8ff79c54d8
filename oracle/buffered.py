"""Buffered per-step decode with periodic rounding (float64 reference).

Test infrastructure only, like the rest of ``oracle/``.

The serving form of periodic rounding: each decode step brings one token per
state; the token goes into a small buffer of the tokens since the last encode,
and every k-th token the state is updated in high precision and re-encoded
('PACE: four-bit recurrent state by rounding less often', flowchart 'Fewer
roundings, less compounded error': new tokens -> small buffer -> every k
tokens a chunked high-precision update -> per-column encode -> stored state;
TL;DR point (1)).  The output of a step is read from the high-precision state
the period holds after that token: the stored state decoded, with the buffered
tokens and the new one applied in order (the same reading as ``pace.py``).

Readings where the pages are silent:

* The buffer holds at most k - 1 tokens: the k-th token of a period triggers
  the encode and leaves the buffer empty.
* Each state has its own buffer fill, so states can sit at different phases
  of their periods (a state skipped by a step keeps its buffer).
* ``flush`` ends every partial period early: buffered tokens are applied and
  the state is encoded, as a shorter final period would be.

Adaptive period (``tau`` given; the same page, section 'Research angle',
proposes tying the re-encode to how much the state has changed since the
last one, not to a fixed token count).  Reading taken:

* The update norm of token t is the Frobenius norm of its write into the
  state, ||k_t|| * ||u_t|| with u_t = beta_t (v_t - alpha_t M_{t-1}^T k_t)
  (M_t = alpha_t M_{t-1} + k_t u_t^T); the accumulated norm A is their sum
  over the buffered tokens.
* The threshold is relative: tau * R, with R = ||decode(stored)||_F of the
  state as of its last encode (0 for a zero state).
* A step closes the period (applies the buffer and its own token, encodes)
  when the buffer is full (period - 1 tokens: ``period`` is the maximum
  period) or when A > tau * R already holds for the buffered tokens: the
  decision is taken before the step's own write is known, so a token whose
  write crosses the threshold makes the next token close the period.

This is written as its own loop over the buffer, separately from
``pace.period`` (which applies a whole period in one call); the tests pin the
two against each other.
"""
from __future__ import annotations

import numpy as np

from . import gdn, quant


class Buffered:
    """n states, each with its stored codes and scales and its own buffer."""

    def __init__(self, codes, scales, bits, period: int, tau=None):
        if period < 1:
            raise ValueError("period must be >= 1")
        if tau is not None and not tau > 0:
            raise ValueError("tau must be positive")
        self.codes = np.array(codes, dtype=np.int16)
        self.scales = np.array(scales, dtype=np.float32)
        self.bits = np.broadcast_to(np.asarray(bits), self.codes.shape[:1]).copy()
        self.period = period
        n = self.codes.shape[0]
        self.buf = [[] for _ in range(n)]  # per state: list of (k, v, alpha, beta)
        self.last_pre = [None] * n           # high-precision state of each state's last encode
        self.tau = tau
        self.A = np.zeros(n)                 # accumulated update norm of the buffered tokens
        self.R = np.array([self._norm(i) for i in range(n)])

    def _norm(self, i: int) -> float:
        return float(np.linalg.norm(quant.decode(self.codes[i], self.scales[i])))

    def closes(self, i: int) -> bool:
        """Whether the next token of state i ends its period."""
        if len(self.buf[i]) + 1 == self.period:
            return True
        return self.tau is not None and self.A[i] > self.tau * self.R[i]

    def margin(self, i: int) -> float:
        """A - tau R relative to tau R (how far the adaptive decision is from its threshold)."""
        t = self.tau * self.R[i]
        return (self.A[i] - t) / t if t > 0 else np.inf

    @property
    def fill(self) -> np.ndarray:
        return np.array([len(b) for b in self.buf])

    def _state(self, i: int) -> np.ndarray:
        """Stored state i decoded, with its buffered tokens applied in order."""
        M = quant.decode(self.codes[i:i + 1], self.scales[i:i + 1])
        for k, v, a, b in self.buf[i]:
            M = gdn.step(M, np.zeros_like(k)[None], k[None], v[None], np.array([a]), np.array([b]))[0]
        return M

    def _encode(self, i: int, M: np.ndarray) -> None:
        c, s = quant.encode(M, self.bits[i:i + 1])
        self.codes[i], self.scales[i] = c[0], s[0]
        self.last_pre[i] = M[0]
        self.buf[i] = []
        self.A[i] = 0.0
        self.R[i] = self._norm(i)

    def step(self, q, k, v, alpha, beta, active=None, decide=None) -> np.ndarray:
        """One token per state: q, k [n, d_k], v [n, d_v], alpha, beta [n]
        (float64 values); active [n] bool or None (all).  ``decide`` [n] bool,
        if given, replaces the adaptive decision of each state (for callers
        matching another implementation where A sits on the threshold).
        Returns the outputs [n, d_v] (NaN for inactive states)."""
        n = self.codes.shape[0]
        act = np.ones(n, dtype=bool) if active is None else np.asarray(active, dtype=bool)
        out = np.full((n, v.shape[1]), np.nan)
        for i in np.nonzero(act)[0]:
            M0 = self._state(i)
            M, o = gdn.step(M0, q[i][None], k[i][None], v[i][None], np.array([alpha[i]]),
                            np.array([beta[i]]))
            out[i] = o[0]
            close = self.closes(i) if decide is None else bool(decide[i])
            if close:
                self._encode(i, M)
            else:
                u = beta[i] * (v[i] - alpha[i] * (k[i] @ M0[0]))
                self.A[i] += np.linalg.norm(k[i]) * np.linalg.norm(u)
                self.buf[i].append((np.array(k[i]), np.array(v[i]), float(alpha[i]), float(beta[i])))
        return out

    def flush(self) -> None:
        """Apply and encode every non-empty buffer (a shorter final period)."""
        for i in range(self.codes.shape[0]):
            if self.buf[i]:
                self._encode(i, self._state(i))
