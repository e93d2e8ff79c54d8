"""Period decode on the GPU against the float64 oracle (through the C ABI)."""
import dataclasses

import numpy as np
import pytest

from linear_attn_decode_pace_amd import inputs
from tests.gpu_cases import default_calls, run_case

pytestmark = pytest.mark.gpu


def test_tiny_full_run():
    # B=4, H=2, d=64, period 4, 64 decode steps, float32 inputs, all heads 4-bit
    w = inputs.TINY
    r = run_case(w, 0, default_calls(w))
    assert r["tiles"] == 8 and r["calls"] == 16


def test_bf16_mixed_ragged():
    # odd batch and head counts, 2 of 5 heads at 8 bits, outlier value channels,
    # and a short final call (a shorter last period)
    w = inputs.ragged("ragged-mixed", 101, B=3, H=5, n_int8=2, n_outliers=8, steps=29)
    calls = default_calls(w, 3) + [(24, 29)]
    run_case(w, 1, calls)


def test_bf16_d64_mixed():
    w = inputs.ragged("d64-mixed", 102, B=5, H=4, dk=64, dv=64, n_int8=1, steps=24)
    run_case(w, 2, default_calls(w))


@pytest.mark.parametrize("period", [1, 2, 4, 8, 16])
def test_period_sweep_small(period):
    # the period sweep of the 256-sequence workload, on a 6-sequence batch
    w = inputs.SWEEP.replace(B=6, period=period, steps=16)
    run_case(w, 3, default_calls(w), label=f"sweep-k{period}")


def test_all_heads_int8():
    w = inputs.ragged("all8", 103, B=2, H=3, n_int8=3, steps=16)
    run_case(w, 4, default_calls(w))


def test_f32_inputs_d128():
    w = inputs.ragged("f32-d128", 104, B=2, H=3, n_int8=1, dtype=inputs.DT_F32, steps=16)
    run_case(w, 5, default_calls(w))


def test_long_periods_ragged():
    # calls of 9..16 tokens (the 16-token chunk kernel) interleaved with
    # shorter ones, odd batch and head counts, 2 of 5 heads at 8 bits
    w = inputs.ragged("long-periods", 105, B=3, H=5, n_int8=2, n_outliers=8, period=16, steps=64)
    calls = [(0, 16), (16, 25), (25, 37), (37, 45), (45, 58), (58, 64)]
    run_case(w, 6, calls)


def test_d64_long_periods():
    w = inputs.ragged("d64-long", 106, B=4, H=4, dk=64, dv=64, n_int8=1, period=16, steps=48)
    run_case(w, 7, [(0, 16), (16, 26), (26, 42), (42, 48)])


def _vanishing_alpha(value):
    # every token of the even sequences decays by `value`: over a period the
    # product gamma_C falls below float32's normal range (or to zero), so the
    # fused kernels take their below-normal-decay branch for those tiles
    def hook(ci, tok):
        a = tok.alpha.copy()
        a[:, 0::2] = np.float32(value)
        return dataclasses.replace(tok, alpha=a)
    return hook


@pytest.mark.parametrize("period,value", [(8, 1e-5), (16, 1e-5), (8, 2e-5)])
def test_vanishing_decay(period, value):
    # period 8 at 1e-5: gamma_C = 1e-40 (a float32 subnormal); period 16:
    # 1e-80 (zero in float32); 2e-5 at period 8: gamma_C = 2.6e-38 is still
    # normal, but gamma_C s falls below float32's normal range
    w = inputs.ragged(f"vanish-k{period}", 107, B=4, H=3, n_int8=1, period=period, steps=2 * period)
    run_case(w, 8, default_calls(w), tok_hook=_vanishing_alpha(value),
             label=f"vanish-k{period}-{value:g}")


def test_padded_periods_vanishing_int8():
    # calls of 9, 11 and 15 tokens (the 16-token kernel pads them with 7, 5
    # and 1 identity tokens that repeat the last real token's inputs), all
    # heads at 8 bits, and the even sequences decaying by 1e-5 per token
    # (the below-normal-decay branch)
    w = inputs.ragged("pad-vanish8", 108, B=4, H=3, n_int8=3, period=16, steps=35)
    run_case(w, 9, [(0, 9), (9, 20), (20, 35)], tok_hook=_vanishing_alpha(1e-5), label="pad-vanish8")


def test_d64_padded_periods():
    # d = 64 (two k-slices per column block) with 9-, 15- and 9-token calls
    w = inputs.ragged("d64-pad", 109, B=3, H=4, dk=64, dv=64, n_int8=2, period=16, steps=33)
    run_case(w, 10, [(0, 9), (9, 24), (24, 33)])


@pytest.mark.parametrize("dv", [48, 80])
def test_dv_differs_from_dk(dv):
    # d_v != d_k (the per-column kernels) with column blocks that do not fill
    # a wavefront (48 columns) or end part way into one (80), mixed heads,
    # column outliers, and a short final call
    w = inputs.ragged(f"dv{dv}", 108, B=3, H=3, dk=128, dv=dv, n_int8=1, n_outliers=4, steps=21)
    run_case(w, 9, default_calls(w, 2) + [(16, 21)])
