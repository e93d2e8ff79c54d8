"""Pins of the oracle's column-scaled quantizer (oracle/quant.py)."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st
from hypothesis.extra import numpy as hnp

from oracle import quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_rint_is_round_half_even():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 6.5])
    assert np.rint(x).tolist() == [0, 2, 2, -0, -2, -2, 4, 6]


@pytest.mark.parametrize("bits", [4, 8])
def test_constructed_exact_ties_go_to_even(bits):
    qm = quant.qmax(bits)
    s = np.float32(0.0123)
    s64 = float(s)
    # column absmax is exactly qmax * s, so the encoded scale is exactly s
    halves = np.arange(-qm + 0.5, qm - 0.5 + 1e-9, 1.0)
    col = np.concatenate([[qm * s64], halves * s64])
    M = col[None, :, None]
    c, sc = quant.encode(M, bits)
    assert sc[0, 0] == s
    expect = np.rint(halves)               # even neighbour
    assert np.all(expect % 2 == 0)
    assert c[0, 1:, 0].tolist() == expect.astype(int).tolist()
    assert c[0, 0, 0] == qm


@pytest.mark.parametrize("bits", [4, 8])
def test_zero_column(bits):
    M = np.zeros((1, 8, 3))
    M[0, 2, 1] = 0.5
    c, s = quant.encode(M, bits)
    assert s[0, 0] == 0 and s[0, 2] == 0
    assert np.all(c[0, :, 0] == 0) and np.all(c[0, :, 2] == 0)
    assert c[0, 2, 1] == quant.qmax(bits)


def _check_invariants(M, bits):
    qm = quant.qmax(bits)
    c, s = quant.encode(M, bits)
    D = quant.decode(c, s)
    s64 = s.astype(np.float64)[..., None, :]
    # round-trip error at most half a step (plus float64 rounding of the quotient)
    assert np.all(np.abs(M - D) <= 0.5 * s64 * (1 + 1e-12) + 1e-300)
    assert np.all(np.abs(c) <= qm)
    nz = np.max(np.abs(M), axis=-2) > 0
    reach = np.max(np.abs(c), axis=-2) == qm
    assert np.all(reach[nz])
    # re-encoding a decoded state gives the same codes and the scale within 1 ulp
    c2, s2 = quant.encode(D, bits)
    assert np.array_equal(c2, c)
    ulp = np.spacing(s)
    assert np.all(np.abs(s2.astype(np.float64) - s) <= ulp)
    return c, s


@settings(max_examples=60, deadline=None)
@given(hnp.arrays(np.float64, (2, 6, 5),
                  elements=st.floats(-1e3, 1e3, allow_nan=False, allow_infinity=False)
                  .filter(lambda x: x == 0 or abs(x) > 1e-20)),
       st.sampled_from([4, 8]))
def test_quantizer_invariants_property(M, bits):
    _check_invariants(M, bits)


@pytest.mark.parametrize("bits", [4, 8])
def test_quantizer_invariants_gaussian(bits):
    rng = np.random.default_rng(7)
    M = rng.standard_normal((8, 64, 64)) * rng.uniform(0.01, 10, (8, 1, 64))
    _check_invariants(M, bits)


def test_scale_is_absmax_over_qmax_in_float32():
    rng = np.random.default_rng(8)
    M = rng.standard_normal((3, 16, 4))
    for bits in (4, 8):
        _, s = quant.encode(M, bits)
        a = np.max(np.abs(M), axis=-2)
        assert np.array_equal(s, (a / quant.qmax(bits)).astype(np.float32))


def test_per_tile_bits():
    rng = np.random.default_rng(9)
    M = rng.standard_normal((2, 16, 4))
    c, s = quant.encode(M, np.array([4, 8]))
    c4, s4 = quant.encode(M[:1], 4)
    c8, s8 = quant.encode(M[1:], 8)
    assert np.array_equal(c[:1], c4) and np.array_equal(c[1:], c8)
    assert np.array_equal(s[:1], s4) and np.array_equal(s[1:], s8)


def test_tie_distance():
    x = np.array([0.5, 1.0, -2.5, 3.25, 0.4999])
    np.testing.assert_allclose(quant.tie_distance(x), [0, 0.5, 0, 0.25, 1e-4], atol=1e-12)


def test_storage_ratios_against_the_pages():
    with open(os.path.join(GOLDEN, "storage_ratios.json")) as f:
        g = {r["name"]: r for r in json.load(f)["ratios"]}
    d = 128
    int4 = quant.tile_bytes(d, d, 4)
    int8 = quant.tile_bytes(d, d, 8)
    fp16 = d * d * 2
    assert int4 == 8192 + 512 and int8 == 16384 + 512
    r = g["int4_vs_fp16"]
    assert abs(int4 / fp16 - r["printed"]) <= r["tolerance"]
    r = g["int4_vs_int8"]
    assert abs(int4 / int8 - r["printed"]) <= r["tolerance"]
    r = g["mixed_4_8_vs_int8"]
    mix = r["mix"]
    ratio = (mix["heads4"] * int4 + mix["heads8"] * int8) / ((mix["heads4"] + mix["heads8"]) * int8)
    assert abs(ratio - r["printed"]) <= r["tolerance"]
    assert abs(ratio - 1344 / 2112) < 1e-12


def test_roundtrip_error_hand_computed():
    # 4 bits; column 0: absmax 7 -> s = 1, 3.5 ties to 4 (error 0.5);
    # column 1: zero; column 2: absmax 7/8 -> s = 1/8, -1/16 ties to -0
    M = np.array([[7.0, 0.0, -1 / 16],
                  [3.5, 0.0, 7 / 8]])[None]
    e, r = quant.roundtrip_error(M, 4)
    assert e.tolist() == [0.25 + 1 / 256]
    assert r.tolist() == [49 + 12.25 + 1 / 256 + 49 / 64]
    # 8 bits: s = 1, 0.5 -> 0 and 1.5 -> 2 (both ties to even)
    e8, r8 = quant.roundtrip_error(np.array([[127.0], [0.5], [1.5]])[None], 8)
    assert e8.tolist() == [0.5] and r8.tolist() == [16129 + 0.25 + 2.25]


@pytest.mark.parametrize("bits", [4, 8])
def test_roundtrip_error_bounds(bits):
    rng = np.random.default_rng(5)
    M = rng.standard_normal((6, 32, 16)) * rng.uniform(0.1, 10, (6, 1, 16))
    e, r = quant.roundtrip_error(M, bits)
    c, s = quant.encode(M, bits)
    # every entry within half a step of its code: err <= d_k * sum_j s_j^2 / 4
    assert np.all(e <= 32 * np.sum(s.astype(np.float64) ** 2, axis=-1) / 4 * (1 + 1e-12))
    assert np.all(e > 0) and np.allclose(r, np.sum(M * M, axis=(1, 2)))
    # a decoded state encodes without error
    e2, _ = quant.roundtrip_error(quant.decode(c, s), bits)
    assert np.all(e2 == 0)


def test_quotients_constructed_values():
    # scales differ per column and the state is not square, so a quotient taken
    # against the wrong axis's scale, or against a recomputed absmax, fails
    s = np.array([0.0123, 0.5, 3.0e-4], dtype=np.float32)
    x = np.array([[2.5, -7.0, 0.5],
                  [-1.5, 6.5, 127.0],
                  [0.0, 3.0, -126.5],
                  [4.0, -0.5, 1.0]])
    M = (x * s.astype(np.float64)[None, :])[None]      # exact: x has few significant bits
    got = quant.quotients(M, s[None])
    assert got.shape == (1, 4, 3)
    assert np.array_equal(got[0], x)
    # the given scales are used as they are: twice the scale halves the quotient
    assert np.array_equal(quant.quotients(M, 2 * s[None])[0], x / 2)
    # a zero scale gives zero quotients whatever the state holds
    z = s.copy()
    z[1] = 0
    got = quant.quotients(M, z[None])
    assert np.all(got[0, :, 1] == 0) and np.array_equal(got[0, :, [0, 2]], x[:, [0, 2]].T)


def test_quotients_keep_float64_precision_near_ties():
    # a quotient 1e-10 away from a half-integer: its tie distance must come out
    # as 1e-10 (a float32 quotient would report 0 or ~1e-7)
    s = np.float32(0.0123)
    eps = 1e-10
    n = np.array([0.5, 2.5, -3.5, 6.5])
    M = ((n + eps) * float(s))[None, :, None]
    d = quant.tie_distance(quant.quotients(M, np.array([[s]])))
    np.testing.assert_allclose(d[0, :, 0], eps, rtol=1e-3)


@pytest.mark.parametrize("bits", [4, 8])
def test_quotients_round_to_the_encoded_codes(bits):
    # encode's codes are the clamped nearest-even rounding of the quotients
    # against its own stored scales
    rng = np.random.default_rng(11)
    M = rng.standard_normal((5, 32, 16)) * rng.uniform(0.01, 10, (5, 1, 16))
    M[0, :, 3] = 0
    c, s = quant.encode(M, bits)
    qm = quant.qmax(bits)
    assert np.array_equal(np.clip(np.rint(quant.quotients(M, s)), -qm, qm).astype(np.int16), c)
