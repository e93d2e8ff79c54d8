"""FP8 write window over a low-bit state (float64 reference, test infrastructure only).

A variant of the buffer from another paper on the pages: '低比特量化新突破：
GGA+PW让线性注意力长文本生成更准更短', section 'PW：让近期写入走“纯净通道”'
(pure-write sliding window): the most recent writes are kept apart from the
low-bit history as FP8 vector pairs, take part in every state transition, and
are merged into the low-bit history only when they leave the window.

Readings where the page is silent:

* A write is the rank-one update of the delta rule written as
  M_t = alpha_t M_{t-1} + k_t u_t^T with u_t = beta_t (v_t - alpha_t M_{t-1}^T k_t)
  (the same recurrence as gdn.step); the pair kept is (k_t, u_t).
* "Taking part in the transition" is then the scalar decay alpha_t applied to
  every window entry and to the history; it is carried as one float64 factor
  per entry (delta) and one for the history (lam), so stored vectors are
  never re-rounded.
* FP8 is OCP E4M3 (bias 7, 3 mantissa bits, subnormal quantum 2^-9, largest
  finite 448); each vector has one float32 scale s = absmax / 448 (0 for a
  zero vector) and its codes are x / s (float32 division) clamped to +-448 and
  rounded to the nearest E4M3 value, ties to even.
* The history is stored with the column quantizer of quant.py and the head's
  bit width; when the window already holds S entries, the oldest leaves after
  the step: history <- encode(lam * decode(history) + delta_o * k_o u_o^T),
  lam <- 1.
* The output of a step is read from the high-precision state after its own
  exact write: o_t = (alpha_t M_{t-1} + k_t u_t^T)^T q_t, with M_{t-1} built
  from the stored history and the stored (FP8) window.
"""
from __future__ import annotations

import math

import numpy as np

from . import quant

E4M3_MAX = 448.0


def e4m3_encode_value(x: float) -> int:
    """Nearest E4M3 code (ties to even) of a float with |x| <= 448."""
    sign = 0x80 if (x < 0 or (x == 0 and math.copysign(1.0, x) < 0)) else 0
    a = abs(x)
    if a == 0:
        return sign
    e = math.floor(math.log2(a))
    if e < -6:
        m = int(np.rint(a / 2.0 ** -9))           # subnormal quantum 2^-9
        return sign | m                            # m = 8 is the smallest normal
    m = int(np.rint(a / 2.0 ** (e - 3)))          # 8 <= m <= 16
    if m == 16:
        e, m = e + 1, 8
    if e > 8 or (e == 8 and m > 15):
        raise ValueError("beyond the largest E4M3 value")
    return sign | ((e + 7) << 3) | (m - 8)


def e4m3_decode_value(c: int) -> float:
    s = -1.0 if c & 0x80 else 1.0
    E, M = (c >> 3) & 15, c & 7
    if E == 15 and M == 7:
        raise ValueError("NaN code")
    if E == 0:
        return s * M * 2.0 ** -9
    return s * (8 + M) * 2.0 ** (E - 10)


def fp8_vector(x: np.ndarray):
    """(codes uint8 [n], float32 scale) of one vector (float64 values)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    s = np.float32(amax / np.float32(E4M3_MAX))
    if s == 0:
        return np.zeros(x32.shape, dtype=np.uint8), np.float32(0)
    q = np.clip(x32 / s, -np.float32(E4M3_MAX), np.float32(E4M3_MAX))
    return np.array([e4m3_encode_value(float(v)) for v in q], dtype=np.uint8), s


def fp8_decode(codes: np.ndarray, s) -> np.ndarray:
    return np.array([e4m3_decode_value(int(c)) for c in codes]) * float(s)


class Window:
    """n states: low-bit history (codes, scales, bit width) and an FP8 window of S writes."""

    def __init__(self, codes, scales, bits, S: int):
        if S < 1:
            raise ValueError("window must hold at least one write")
        self.codes = np.array(codes, dtype=np.int16)
        self.scales = np.array(scales, dtype=np.float32)
        n = self.codes.shape[0]
        self.bits = np.broadcast_to(np.asarray(bits), (n,)).copy()
        self.S = S
        self.lam = np.ones(n)
        self.win = [[] for _ in range(n)]  # per state, oldest first: [kc, ks, uc, us, delta]
        self.last_pre = [None] * n         # high-precision history of each state's last encode

    def state(self, i: int) -> np.ndarray:
        """The state M of state i as stored: lam * history + sum of decayed FP8 writes."""
        M = self.lam[i] * quant.decode(self.codes[i], self.scales[i])
        for kc, ks, uc, us, delta in self.win[i]:
            M = M + delta * np.outer(fp8_decode(kc, ks), fp8_decode(uc, us))
        return M

    def step(self, q, k, v, alpha, beta) -> np.ndarray:
        """One token per state (float64 values): q, k [n, d_k], v [n, d_v],
        alpha, beta [n].  Returns the outputs [n, d_v]."""
        n = self.codes.shape[0]
        out = np.empty((n, v.shape[1]))
        for i in range(n):
            M = self.state(i)
            u = beta[i] * (v[i] - alpha[i] * (k[i] @ M))
            out[i] = (alpha[i] * M + np.outer(k[i], u)).T @ q[i]
            self.lam[i] *= alpha[i]
            for e in self.win[i]:
                e[4] *= alpha[i]
            kc, ks = fp8_vector(k[i])
            uc, us = fp8_vector(u)
            self.win[i].append([kc, ks, uc, us, 1.0])
            if len(self.win[i]) > self.S:
                self._merge_oldest(i)
        return out

    def _merge_oldest(self, i: int) -> None:
        kc, ks, uc, us, delta = self.win[i].pop(0)
        H = self.lam[i] * quant.decode(self.codes[i], self.scales[i]) + \
            delta * np.outer(fp8_decode(kc, ks), fp8_decode(uc, us))
        c, s = quant.encode(H[None], self.bits[i:i + 1])
        self.codes[i], self.scales[i] = c[0], s[0]
        self.lam[i] = 1.0
        self.last_pre[i] = H

    def flush(self) -> None:
        """Merge every window entry into the history (oldest first), one encode
        per state with a non-empty window."""
        for i in range(self.codes.shape[0]):
            if not self.win[i]:
                continue
            H = self.lam[i] * quant.decode(self.codes[i], self.scales[i])
            for kc, ks, uc, us, delta in self.win[i]:
                H = H + delta * np.outer(fp8_decode(kc, ks), fp8_decode(uc, us))
            c, s = quant.encode(H[None], self.bits[i:i + 1])
            self.codes[i], self.scales[i] = c[0], s[0]
            self.lam[i] = 1.0
            self.win[i] = []
            self.last_pre[i] = H
