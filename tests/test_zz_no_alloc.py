"""pace_quant_stats_static, the statistics entry point that allocates no
device memory (its counter and error sums live in a fixed array per device),
through the C ABI against pace_quant_stats on the same handles: two calls in
a row, the second on a smaller handle, so a stale counter or stale sums left
by the first call would show; then the larger handle again."""
import ctypes

import pytest

from linear_attn_decode_pace_amd import inputs

pytestmark = pytest.mark.gpu


def _stats(fn, handle):
    from linear_attn_decode_pace_amd import pace

    s = pace.pace_stats()
    rc = fn(handle, ctypes.byref(s), None)
    assert rc == pace.PACE_OK, pace.pace_last_error()
    return s


def _same(a, b, heads):
    from linear_attn_decode_pace_amd import pace

    for name, _ in pace.pace_stats._fields_:
        if name in ("err_sq", "ref_sq"):
            assert list(getattr(a, name))[:heads] == list(getattr(b, name))[:heads], name
        else:
            assert getattr(a, name) == getattr(b, name), name


def test_static_stats_match_allocating_stats_twice():
    from linear_attn_decode_pace_amd import pace, runtime

    # larger handle: error tracking, a decoded period (no zero columns)
    wb = inputs.ragged("nz-big", 300, B=6, H=7, n_int8=2, n_outliers=4, steps=8)
    big = runtime.State(wb, inputs.head_bits(wb, 0), pace.PACE_INIT_F32, runtime.warmup_state(wb, 0),
                        flags=pace.PACE_STATS_ERR)
    tok = runtime.DeviceTokens(inputs.tokens(wb, 0, inputs.SEG_DECODE, 0, 8))
    big.decode(tok, runtime.out_buffer(wb, 8))
    # smaller handle: its initial encode, with five zero columns per state
    ws = inputs.ragged("nz-small", 301, B=2, H=3, n_int8=1, steps=8)
    M0 = runtime.warmup_state(ws, 0)
    M0[..., :5] = 0.0
    small = runtime.State(ws, inputs.head_bits(ws, 0), pace.PACE_INIT_F32, M0, flags=pace.PACE_STATS_ERR)

    first = _stats(pace.LIB.pace_quant_stats_static, big.handle)
    _same(first, _stats(pace.LIB.pace_quant_stats, big.handle), wb.H)
    assert first.err_tracked == 1 and first.zero_columns == 0 and sum(first.err_sq[:wb.H]) > 0
    second = _stats(pace.LIB.pace_quant_stats_static, small.handle)
    _same(second, _stats(pace.LIB.pace_quant_stats, small.handle), ws.H)
    assert second.zero_columns == ws.B * ws.H * 5 and sum(second.err_sq[:ws.H]) > 0
    _same(_stats(pace.LIB.pace_quant_stats_static, big.handle), first, wb.H)
    big.free()
    small.free()
