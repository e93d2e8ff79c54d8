"""Column-scaled symmetric quantizer (float64 reference).

Follows 'PACE: A New 4-Bit Recurrent State Quantization Method That Makes
Linear Attention Models More Memory-Efficient', section 'Channel-Aligned
Encoding: Exploiting State Column Structure' (one quantization scale shared by
all entries of a state column), and 'PACE: four-bit recurrent state by
rounding less often', TL;DR point (2) and the flowchart's "4-bit encode,
per-column scales".  The pages do not print the scale formula; the reading
used here is the plain symmetric absmax one:

    qmax = 2**(bits-1) - 1            (7 for 4 bits, 127 for 8 bits)
    a_j  = max_i |M[i, j]|            (column j = value channel j)
    s_j  = a_j / qmax rounded to float32 (nearest even); s_j = 0 if a_j = 0
    c_ij = clamp(rint(M[i, j] / s_j), -qmax, qmax)   (rint = nearest even)
    M'   = c_ij * s_j

The quotient is taken against the stored float32 scale, so both sides
dequantize with the same number.

Pinned by tests/test_oracle_quant.py: round-trip error <= s/2, |c| <= qmax,
every non-zero column reaches +-qmax, exact constructed ties go to the even
neighbour, re-encoding a decoded state is the identity on the codes, and the
storage closed forms against the ratios the pages print.
"""
from __future__ import annotations

import numpy as np


def qmax(bits: int) -> int:
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    return (1 << (bits - 1)) - 1


def _qmax_per_tile(bits, n_lead_shape):
    b = np.asarray(bits)
    q = np.where(b == 8, 127, np.where(b == 4, 7, -1)).astype(np.float64)
    if np.any(q < 0):
        raise ValueError("bits must be 4 or 8")
    return np.broadcast_to(q, n_lead_shape)


def encode(M: np.ndarray, bits):
    """Quantize states M [..., d_k, d_v] (float64) column by column.

    ``bits`` is a scalar or an array broadcastable to M.shape[:-2].
    Returns (codes int16 [..., d_k, d_v], scales float32 [..., d_v]).
    """
    M = np.asarray(M, dtype=np.float64)
    qm = _qmax_per_tile(bits, M.shape[:-2])[..., None]          # [..., 1]
    a = np.max(np.abs(M), axis=-2)                               # [..., d_v]
    s = (a / qm).astype(np.float32)
    s64 = s.astype(np.float64)[..., None, :]                     # [..., 1, d_v]
    safe = np.where(s64 > 0, s64, 1.0)
    x = np.where(s64 > 0, M / safe, 0.0)
    lim = qm[..., None]
    c = np.clip(np.rint(x), -lim, lim).astype(np.int16)
    return c, s


def decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Dequantize: M[i, j] = c_ij * s_j, exact in float64."""
    return codes.astype(np.float64) * scales.astype(np.float64)[..., None, :]


def quotients(M: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """M / s per entry against the given float32 scales (0 where s = 0)."""
    s64 = np.asarray(scales, dtype=np.float64)[..., None, :]
    safe = np.where(s64 > 0, s64, 1.0)
    return np.where(s64 > 0, np.asarray(M, dtype=np.float64) / safe, 0.0)


def roundtrip_error(M: np.ndarray, bits):
    """Squared round-trip error of encoding states M [..., d_k, d_v]:
    returns (sum (M - decode(encode(M)))**2, sum M**2), each summed over the
    last two axes (one value per state).  Their ratio is the state's relative
    squared quantization error under the column quantizer above."""
    M = np.asarray(M, dtype=np.float64)
    c, s = encode(M, bits)
    d = M - decode(c, s)
    return np.sum(d * d, axis=(-2, -1)), np.sum(M * M, axis=(-2, -1))


def tie_distance(x: np.ndarray) -> np.ndarray:
    """Distance of each quotient from the nearest half-integer (rounding tie)."""
    return np.abs(np.abs(x - np.floor(x)) - 0.5)


def tile_bytes(d_k: int, d_v: int, bits: int) -> int:
    """Stored bytes of one (sequence, head) state: codes plus float32 scales."""
    return d_k * d_v * bits // 8 + 4 * d_v
