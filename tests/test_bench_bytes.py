"""The byte counts bench.py divides by time (CPU only).

Per-tile figures at d = 128, C = 8, bf16 are worked out by hand: a 4-bit tile
reads and writes 8,192 B of codes and 512 B of scales (17,408 B), and its 8
tokens move 8 x (3 x 256 + 8 + 512) = 10,304 B, 27,712 B in all; an 8-bit tile
moves 2 x (16,384 + 512) + 10,304 = 44,096 B.
"""
import pytest

torch = pytest.importorskip("torch")

import bench  # noqa: E402
from linear_attn_decode_pace_amd import inputs  # noqa: E402


def test_period_bytes_headline_by_hand():
    w = inputs.HEADLINE
    bits = inputs.head_bits(w, 0)
    n8 = int((bits == 8).sum())
    assert n8 == 4
    assert bench.algorithmic_bytes(w, w.period, bits) == w.B * ((w.H - n8) * 27712 + n8 * 44096)
    assert bench.algorithmic_bytes(w, w.period, bits) == 2084569088


def test_exact_step_bytes_match_the_period_model():
    # a whole fixed period, call by call, equals the per-call mean of the model
    w = inputs.HEADLINE.replace(B=8)
    bits = inputs.head_bits(w, 0)
    fill = torch.zeros((w.B, w.H), dtype=torch.int32)
    total = 0.0
    for f in range(w.period):
        closed = torch.full((w.B, w.H), f == w.period - 1)
        total += bench.step_bytes_exact(w, bits, fill, closed)
        fill = torch.zeros_like(fill) if f == w.period - 1 else fill + 1
    assert total / w.period == pytest.approx(bench.algorithmic_bytes_step(w, bits), rel=1e-12)


def test_exact_step_bytes_per_state():
    # one state of each width, one closing its period after 3 buffered tokens,
    # the other appending its 6th token: counted by hand
    w = inputs.HEADLINE.replace(B=1, H=2)
    bits = [4, 8]
    fill = torch.tensor([[3, 5]], dtype=torch.int32)
    closed = torch.tensor([[True, False]])
    st4, st8 = 128 * 128 // 2 + 512, 128 * 128 + 512
    buf, io = 2 * 128 * 2 + 8, 3 * 128 * 2 + 8 + 512
    want = (st4 + 3 * buf + io + st4) + (st8 + 5 * buf + io + buf)
    assert bench.step_bytes_exact(w, bits, fill, closed) == want
