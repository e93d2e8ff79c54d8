"""Comparison of the HIP path against the float64 oracle.

Tolerances (relative L2 unless stated):

* outputs o_t per (sequence, head) tile: 2e-3; float32 arithmetic in fact
  reaches ~1e-6, so a tighter diagnostic bar of 1e-4 is asserted as well;
* scales: 1e-5 relative, zero equals zero;
* codes: equal, except +-1 flips where the oracle's quotient M / s lies within
  1e-3 of a half-integer (a rounding tie that float32 and float64 may resolve
  differently), on at most 0.1% of the entries (for a merge of the FP8 write
  window, on at most the entries the oracle holds within 1e-5 of a tie: a
  column dominated by an E4M3 write has its quotients on exact half-integers);
* dequantized state: 2e-3 per tile and aggregated over all checked tiles,
  with the entries of allowed flips masked.  A single allowed 4-bit flip moves
  one entry by a whole code step (1/7 of its column's largest entry), which by
  itself can exceed 2e-3 of the aggregate norm; the unmasked error is reported
  but not asserted, since asserting it would forbid the flips allowed above.

Parity is checked two ways.  *Transition validity*: each period is replayed by
the oracle from the state the GPU stored at the end of the previous period
(after that state itself passed the checks), so every transition the GPU makes
is held to the bars above even after a legitimate tie flip has made the two
trajectories differ by a code step.  *Free-running*: an independent oracle
trajectory from the oracle's own warm-up; its outputs and codes must match the
GPU's bit-for-bit modulo ties for every tile in which no tie flip has happened
yet (a tile that flipped is reported and then left to the transition check).
"""
from __future__ import annotations

import dataclasses

import numpy as np

from oracle import quant

REL_OUT = 2e-3
REL_OUT_TIGHT = 1e-4
REL_SCALE = 1e-5
REL_STATE = 2e-3
TIE_TOL = 1e-3
MAX_FLIP_FRAC = 1e-3


def rel_per_tile(x: np.ndarray, ref: np.ndarray, tile_axis: int) -> np.ndarray:
    """Relative L2 error per tile; tiles run along ``tile_axis``."""
    x = np.moveaxis(np.asarray(x, dtype=np.float64), tile_axis, 0)
    ref = np.moveaxis(np.asarray(ref, dtype=np.float64), tile_axis, 0)
    n = x.shape[0]
    num = np.linalg.norm((x - ref).reshape(n, -1), axis=1)
    den = np.linalg.norm(ref.reshape(n, -1), axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def rel(x, ref) -> float:
    d = np.linalg.norm(np.asarray(ref, dtype=np.float64))
    n = np.linalg.norm(np.asarray(x, dtype=np.float64) - ref)
    return float(n / d) if d > 0 else float(n)


@dataclasses.dataclass
class Report:
    flips: int = 0
    entries: int = 0
    max_out: float = 0.0
    max_state_masked: float = 0.0
    state_unmasked: float = 0.0
    max_scale: float = 0.0

    def merge(self, o: "Report") -> "Report":
        return Report(self.flips + o.flips, self.entries + o.entries,
                      max(self.max_out, o.max_out),
                      max(self.max_state_masked, o.max_state_masked),
                      max(self.state_unmasked, o.state_unmasked),
                      max(self.max_scale, o.max_scale))


def check_encoded(codes, scales, ref_codes, ref_scales, M_ref, what="",
                  lattice_ties=False) -> Report:
    """GPU codes/scales against the oracle's encode of M_ref (the high-precision
    state the oracle had just before encoding).  lattice_ties: states whose
    quotients sit on exact rounding ties by construction (FP8 writes merged
    into the history) may flip every such tie, not only 0.1% of entries."""
    codes = np.asarray(codes).astype(np.int16)
    ref_codes = np.asarray(ref_codes).astype(np.int16)
    scales = np.asarray(scales, dtype=np.float64)
    ref_scales = np.asarray(ref_scales, dtype=np.float64)
    rep = Report()
    # scales
    zero_ref = ref_scales == 0
    assert np.array_equal(scales == 0, zero_ref), f"{what}: zero-scale columns differ"
    rs = np.abs(scales - ref_scales) / np.where(zero_ref, 1, ref_scales)
    rep.max_scale = float(rs.max(initial=0))
    assert rep.max_scale <= REL_SCALE, f"{what}: scale rel err {rep.max_scale:.3g}"
    # codes
    diff = codes - ref_codes
    assert np.abs(diff).max(initial=0) <= 1, f"{what}: code differs by more than one step"
    flips = diff != 0
    rep.flips = int(flips.sum())
    rep.entries = int(codes.size)
    if rep.flips:
        x = quant.quotients(M_ref, ref_scales)
        td = quant.tie_distance(x)[flips]
        assert td.max() < TIE_TOL, f"{what}: code flip away from a rounding tie (distance {td.max():.3g})"
    budget = MAX_FLIP_FRAC * rep.entries
    if lattice_ties and rep.flips:
        budget = max(budget, int((quant.tie_distance(quant.quotients(M_ref, ref_scales)) < 1e-5).sum()))
    assert rep.flips <= budget, f"{what}: {rep.flips} flips of {rep.entries}"
    # dequantized state
    D = codes.astype(np.float64) * scales[..., None, :]
    Dr = ref_codes.astype(np.float64) * ref_scales[..., None, :]
    rep.state_unmasked = rel(D, Dr)
    if rep.flips:
        x = quant.quotients(M_ref, ref_scales)
        td_all = quant.tie_distance(x)
        print(f"  {what}: {rep.flips} flips of {rep.entries}; oracle entries within 1e-5/1e-4/1e-3 "
              f"of a tie: {(td_all < 1e-5).sum()}/{(td_all < 1e-4).sum()}/{(td_all < 1e-3).sum()}; "
              f"flip tie distances max {quant.tie_distance(x)[flips].max():.2e}; "
              f"state rel {rep.state_unmasked:.2e}", flush=True)
    Dm = np.where(flips, Dr, D)
    rep.max_state_masked = float(rel_per_tile(Dm, Dr, 0).max(initial=0))
    assert rep.max_state_masked <= REL_STATE, f"{what}: masked state err {rep.max_state_masked:.3g}"
    agg = rel(Dm, Dr)
    assert agg <= REL_STATE, f"{what}: masked aggregate state err {agg:.3g}"
    return rep


def check_outputs(out, ref_out, what="") -> float:
    """Outputs [T, n, d_v] per tile (tile axis 1)."""
    r = rel_per_tile(out, ref_out, 1)
    m = float(r.max(initial=0))
    assert m <= REL_OUT, f"{what}: output rel err {m:.3g} (bar {REL_OUT})"
    assert m <= REL_OUT_TIGHT, f"{what}: output rel err {m:.3g} above float32 expectation {REL_OUT_TIGHT}"
    return m


def tiles(a: np.ndarray) -> np.ndarray:
    """[T, B, H, ...] -> [T, B*H, ...]"""
    return a.reshape((a.shape[0], -1) + a.shape[3:])
