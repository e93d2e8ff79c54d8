"""Seeded synthetic workloads for PACE-style GDN decode.

This module only draws random numbers and shapes them into the inputs
that both sides consume: the CPU oracle (through the tests and the bench's
CPU-baseline leg) and the HIP library (through the binding).  It holds none of
the method's arithmetic: no recurrence, no quantizer, no state.

Recipe (every value is synthetic and seeded):

* q_t, k_t ~ N(0, 1) per element, L2-normalised over d_k (norm taken in
  float64, result rounded to float32), then stored either as float32 or
  rounded to bfloat16 (round to nearest even).
* v_t ~ N(0, 1) per element; for the outlier workloads a seeded set of value
  channels is multiplied by a constant before the final cast, so that some
  state columns carry large entries (the pages observe that large entries of a
  gated-delta state cluster in columns: 'PACE: four-bit recurrent state by
  rounding less often', TL;DR point (2)).
* beta_t = sigmoid(z), alpha_t = exp(-softplus(z)) for z ~ N(0, 1), computed
  in float64 and stored as float32; one scalar per (token, sequence, head).

Random streams are counter-keyed: one Philox stream per
(workload id, seed, segment, block of 8 tokens), drawn over the whole batch in
a fixed order (alpha normals, beta normals, q, k, v).  A period can therefore
be regenerated on its own, and every period length sees the same token
sequence.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence

import numpy as np

TB = 8  # tokens per generation block

SEG_WARMUP = 1
SEG_DECODE = 2
SEG_PROMPT = 3
SEG_OUTLIER = 4

DT_F32 = "f32"
DT_BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and recipe of one synthetic decode workload."""

    name: str
    wid: int                 # workload id, part of every random stream key
    B: int                   # sequences decoding concurrently
    H: int                   # heads of the layer
    dk: int
    dv: int
    period: int              # tokens applied per decode call (k)
    steps: int               # decode steps of the whole run
    dtype: str               # q/k/v storage: "f32" or "bf16"
    n_int8: int = 0          # heads kept at 8 bits (largest mean alpha)
    n_outliers: int = 0      # value channels scaled by `outlier_scale`
    outlier_scale: float = 16.0
    warmup: int = 32         # unquantized warm-up tokens before decode
    prompt: int = 0          # prompt tokens for a prefill hand-off (0 = none)
    prefill_chunk: int = 64

    @property
    def periods(self) -> int:
        return self.steps // self.period

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads the method is measured on.
TINY = Workload("tiny", 0, B=4, H=2, dk=64, dv=64, period=4, steps=64,
                dtype=DT_F32)
SWEEP = Workload("sweep-b256", 1, B=256, H=16, dk=128, dv=128, period=8,
                 steps=256, dtype=DT_BF16)
MIXED = Workload("mixed-b1024", 2, B=1024, H=16, dk=128, dv=128, period=8,
                 steps=512, dtype=DT_BF16, n_int8=4, n_outliers=8)
HEADLINE = Workload("mixed-b4096", 3, B=4096, H=16, dk=128, dv=128, period=8,
                    steps=1024, dtype=DT_BF16, n_int8=4, n_outliers=8)
PREFILL = Workload("prefill-b512", 4, B=512, H=32, dk=128, dv=128, period=16,
                   steps=2048, dtype=DT_BF16, n_int8=8, warmup=0, prompt=4096)

WORKLOADS: Dict[str, Workload] = {w.name: w for w in
                                  (TINY, SWEEP, MIXED, HEADLINE, PREFILL)}


def _rng(w: Workload, seed: int, seg: int, blk: int) -> np.random.Generator:
    ss = np.random.SeedSequence([int(seed), int(w.wid), int(seg), int(blk)])
    return np.random.Generator(np.random.Philox(ss))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even); return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def outlier_channels(w: Workload, seed: int) -> np.ndarray:
    if w.n_outliers == 0:
        return np.zeros(0, dtype=np.int64)
    rng = _rng(w, seed, SEG_OUTLIER, 0)
    return np.sort(rng.choice(w.dv, size=w.n_outliers, replace=False))


@dataclasses.dataclass
class Tokens:
    """Inputs of a run of tokens, laid out [T, B, H, ...] as the library takes them.

    q, k, v are float32 arrays (dtype f32) or uint16 bfloat16 bit patterns
    (dtype bf16); alpha and beta are float32 [T, B, H].
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    dtype: str

    @property
    def T(self) -> int:
        return self.alpha.shape[0]

    def f64(self, name: str) -> np.ndarray:
        """The stored values of one tensor, exactly, as float64."""
        a = getattr(self, name)
        if name in ("q", "k", "v") and self.dtype == DT_BF16:
            a = bf16_to_f32(a)
        return a.astype(np.float64)

    def slice(self, t0: int, t1: int) -> "Tokens":
        return Tokens(self.q[t0:t1], self.k[t0:t1], self.v[t0:t1],
                      self.alpha[t0:t1], self.beta[t0:t1], self.dtype)

    def select(self, b: Sequence[int], h: Sequence[int]) -> "Tokens":
        """Tokens of the (sequence, head) pairs b[i], h[i], as [T, n, 1, ...]."""
        b = np.asarray(b)
        h = np.asarray(h)
        return Tokens(self.q[:, b, h][:, :, None], self.k[:, b, h][:, :, None],
                      self.v[:, b, h][:, :, None], self.alpha[:, b, h][:, :, None],
                      self.beta[:, b, h][:, :, None], self.dtype)


def _block(w: Workload, seed: int, seg: int, blk: int, alpha_only=False):
    rng = _rng(w, seed, seg, blk)
    shp = (TB, w.B, w.H)
    za = rng.standard_normal(shp)
    alpha = np.exp(-np.logaddexp(0.0, za)).astype(np.float32)
    if alpha_only:
        return alpha
    zb = rng.standard_normal(shp)
    beta = (1.0 / (1.0 + np.exp(-zb))).astype(np.float32)
    q = rng.standard_normal(shp + (w.dk,), dtype=np.float32).astype(np.float64)
    k = rng.standard_normal(shp + (w.dk,), dtype=np.float32).astype(np.float64)
    v = rng.standard_normal(shp + (w.dv,), dtype=np.float32)
    q = (q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True))).astype(np.float32)
    k = (k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True))).astype(np.float32)
    oc = outlier_channels(w, seed)
    if oc.size:
        v[..., oc] *= np.float32(w.outlier_scale)
    if w.dtype == DT_BF16:
        q, k, v = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    return q, k, v, alpha, beta


def tokens(w: Workload, seed: int, seg: int, t0: int, t1: int) -> Tokens:
    """Tokens [t0, t1) of one segment (warm-up, decode or prompt)."""
    if t1 <= t0:
        raise ValueError("empty token range")
    b0, b1 = t0 // TB, (t1 + TB - 1) // TB
    parts = [_block(w, seed, seg, blk) for blk in range(b0, b1)]
    cat = [np.concatenate([p[i] for p in parts], axis=0) for i in range(5)]
    lo = t0 - b0 * TB
    sl = slice(lo, lo + (t1 - t0))
    return Tokens(cat[0][sl], cat[1][sl], cat[2][sl], cat[3][sl], cat[4][sl],
                  w.dtype)


def _tokens_job(args):
    return tokens(*args)


def iter_tokens(w: Workload, seed: int, seg: int, ranges, workers: int = 1):
    """Tokens of several ranges [(t0, t1), ...] in order, generated by a
    process pool when workers > 1 (the values do not depend on workers)."""
    jobs = [(w, seed, seg, t0, t1) for t0, t1 in ranges]
    if workers <= 1 or len(jobs) <= 1:
        for j in jobs:
            yield tokens(*j)
        return
    import concurrent.futures as cf
    with cf.ProcessPoolExecutor(max_workers=workers) as ex:
        for tok in ex.map(_tokens_job, jobs):
            yield tok


def concat(parts) -> Tokens:
    parts = list(parts)
    return Tokens(*[np.concatenate([getattr(p, n) for p in parts], axis=0)
                    for n in ("q", "k", "v", "alpha", "beta")], parts[0].dtype)


def decode_period(w: Workload, seed: int, p: int, period: Optional[int] = None) -> Tokens:
    """The tokens of decode period p (period length defaults to the workload's)."""
    c = w.period if period is None else period
    return tokens(w, seed, SEG_DECODE, p * c, (p + 1) * c)


def warmup_tokens(w: Workload, seed: int) -> Tokens:
    return tokens(w, seed, SEG_WARMUP, 0, w.warmup)


def mean_alpha(w: Workload, seed: int) -> np.ndarray:
    """Mean gate per head over the pre-decode tokens (warm-up or prompt), [H]."""
    seg, n = (SEG_PROMPT, w.prompt) if w.prompt else (SEG_WARMUP, w.warmup)
    acc = np.zeros(w.H, dtype=np.float64)
    if n == 0:   # no tokens before decode: every head ties (lowest indices win)
        return acc
    for blk in range((n + TB - 1) // TB):
        a = _block(w, seed, seg, blk, alpha_only=True).astype(np.float64)
        m = min(TB, n - blk * TB)
        acc += a[:m].sum(axis=(0, 1))
    return acc / (n * w.B)


def head_bits(w: Workload, seed: int) -> np.ndarray:
    """Bit width per head: the n_int8 heads with the largest mean gate (slowest
    decay, so rounding error persists longest) get 8 bits, the rest 4.  Ties go
    to the lower head index."""
    bits = np.full(w.H, 4, dtype=np.uint8)
    if w.n_int8:
        m = mean_alpha(w, seed)
        order = np.argsort(-m, kind="stable")
        bits[order[: w.n_int8]] = 8
    return bits


def ragged(name: str, wid: int, **kw) -> Workload:
    """A small custom workload (ragged batch, odd head counts) for tests."""
    base = dict(B=3, H=3, dk=128, dv=128, period=8, steps=16, dtype=DT_BF16)
    base.update(kw)
    return Workload(name, wid, **base)
