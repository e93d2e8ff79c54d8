"""The seeded input generator: determinism, recipe and period independence."""
import numpy as np

from linear_attn_decode_pace_amd import inputs


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.14159], dtype=np.float32)
    got = inputs.bf16_to_f32(inputs.bf16_bits(x))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: goes to the even mantissa (1.0)
    # 1 + 3 * 2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: goes to 1 + 2^-6
    assert got.tolist() == [1.0, 1.0, 1.015625, -2.5, np.float32(3.140625)]


def test_periods_are_regenerated_identically():
    w = inputs.TINY
    whole = inputs.tokens(w, 0, inputs.SEG_DECODE, 0, 16)
    p2 = inputs.decode_period(w, 0, 2)
    for n in ("q", "k", "v", "alpha", "beta"):
        assert np.array_equal(getattr(whole, n)[8:12], getattr(p2, n))


def test_period_length_does_not_change_tokens():
    w = inputs.SWEEP.replace(B=2, H=2)
    a = inputs.decode_period(w, 0, 1, period=16)
    b = inputs.decode_period(w, 0, 7, period=4)
    assert np.array_equal(a.q[-4:], b.q) and np.array_equal(a.alpha[-4:], b.alpha)


def test_recipe():
    w = inputs.MIXED.replace(B=64)
    t = inputs.decode_period(w, 0, 0)
    assert t.q.dtype == np.uint16 and t.alpha.dtype == np.float32
    q = t.f64("q")
    assert np.allclose(np.linalg.norm(q, axis=-1), 1, atol=1e-2)
    assert np.all((t.alpha > 0) & (t.alpha < 1)) and np.all((t.beta > 0) & (t.beta < 1))
    v = t.f64("v")
    oc = inputs.outlier_channels(w, 0)
    assert len(oc) == 8
    rms = np.sqrt(np.mean(v ** 2, axis=(0, 1, 2)))
    others = np.setdiff1d(np.arange(w.dv), oc)
    assert rms[oc].min() > 8 and rms[others].max() < 2


def test_head_bits_largest_mean_alpha():
    w = inputs.MIXED.replace(B=32)
    bits = inputs.head_bits(w, 0)
    m = inputs.mean_alpha(w, 0)
    assert (bits == 8).sum() == 4
    assert m[bits == 8].min() >= m[bits == 4].max()


def test_f32_workload_keeps_f32():
    t = inputs.decode_period(inputs.TINY, 0, 0)
    assert t.q.dtype == np.float32 and t.q.shape == (4, 4, 2, 64)
