"""Per-step buffered decode (pace_decode_step) on the GPU.

Two checks: with every sequence active, steps must give bitwise the outputs
and stored states of period calls fed the same tokens (the fused and the
per-column paths compute the same chunk either way); with seeded activity
masks (sequences at different phases), every step is checked against the
buffered oracle (oracle/buffered.py), whose stored states are re-synchronised
from the GPU's after each checked encode (transition validity, as for period
calls).
"""
import numpy as np
import pytest

from linear_attn_decode_pace_amd import inputs
from oracle import buffered, quant
from tests import parity
from tests.gpu_cases import say, tok_tiles

pytestmark = pytest.mark.gpu

CASES = [
    ("step-k4", dict(B=3, H=5, n_int8=2, n_outliers=8, period=4, steps=16)),      # fused
    ("step-k8-d64", dict(B=4, H=4, dk=64, dv=64, n_int8=1, period=8, steps=16)),  # fused, d = 64
    ("step-f32", dict(B=2, H=3, n_int8=1, dtype=inputs.DT_F32, period=4, steps=12)),  # per-column
    # steps of periods above 8 run the per-column kernel, period calls the
    # 16-token fused kernel: checked against the oracle only
    ("step-k12", dict(B=3, H=3, n_int8=1, period=12, steps=24)),
    # d_v != d_k: the per-column step and flush kernels
    ("step-dv48", dict(B=3, H=3, dv=48, n_int8=1, n_outliers=4, period=4, steps=12)),
]


def _states(w, seed):
    from linear_attn_decode_pace_amd import pace, runtime
    bits = inputs.head_bits(w, seed)
    M0 = runtime.warmup_state(w, seed)
    per = runtime.State(w, bits, pace.PACE_INIT_F32, M0)
    stp = runtime.State(w, bits, pace.PACE_INIT_F32, M0, flags=pace.PACE_STEP_BUFFER)
    return bits, per, stp


@pytest.mark.parametrize("name,kw", CASES[:3] + [CASES[4]])
def test_steps_equal_period_calls(name, kw):
    import torch
    from linear_attn_decode_pace_amd import runtime
    w = inputs.ragged(name, 220, **kw)
    seed = 0
    say(f"[case] steps vs period calls {name}")
    bits, per, stp = _states(w, seed)
    C = w.period
    for p in range(w.steps // C):
        tok = inputs.tokens(w, seed, inputs.SEG_DECODE, p * C, (p + 1) * C)
        dt = runtime.DeviceTokens(tok)
        out_p = runtime.out_buffer(w, C)
        per.decode(dt, out_p)
        raw0 = stp.read_raw()
        for t in range(C):
            out_s = runtime.out_buffer(w, 1)
            stp.step(dt.slice(t, t + 1), out_s)
            assert torch.equal(out_s[0], out_p[t]), f"{name}: period {p} token {t}"
            if t < C - 1:   # mid-period: the stored state is only read
                assert torch.equal(stp.read_raw(), raw0), f"{name}: period {p} token {t} wrote"
        assert torch.equal(stp.read_raw(), per.read_raw()), f"{name}: state after period {p}"
    per.free()
    stp.free()


@pytest.mark.parametrize("name,kw", [CASES[0], CASES[1], CASES[3], CASES[4]])
def test_masked_steps_against_buffered_oracle(name, kw):
    import torch
    from linear_attn_decode_pace_amd import pace, runtime
    w = inputs.ragged(name + "-mask", 221, **kw)
    seed = 1
    say(f"[case] masked steps {name}")
    n = w.B * w.H
    idx = np.arange(n)
    bits = inputs.head_bits(w, seed)
    bits_t = np.tile(bits, w.B).astype(np.int64)
    st = runtime.State(w, bits, pace.PACE_INIT_F32, runtime.warmup_state(w, seed),
                       flags=pace.PACE_STEP_BUFFER)

    def read():
        c, s = st.read_codes()
        return c.reshape(n, w.dk, w.dv).cpu().numpy(), s.reshape(n, w.dv).cpu().numpy()

    codes, scales = read()
    ref = buffered.Buffered(codes, scales, bits_t, w.period)
    rng = np.random.default_rng(5)
    T = w.steps + w.period // 2
    encodes = 0
    for t in range(T):
        act = rng.uniform(size=w.B) < 0.7
        if t < 2:
            act[:] = True
        tok = inputs.tokens(w, seed, inputs.SEG_DECODE, t, t + 1)
        out = runtime.out_buffer(w, 1).fill_(np.nan)
        st.step(runtime.DeviceTokens(tok), out,
                torch.as_tensor(act.astype(np.uint8), device="cuda"))
        q, k, v, a, b = [x[0] for x in tok_tiles(tok, idx, w.H)]
        fill_before = ref.fill
        act_t = np.repeat(act, w.H)
        o_ref = ref.step(q, k, v, a, b, act_t)
        o = out.reshape(n, w.dv).cpu().numpy()
        assert np.all(np.isnan(o[~act_t])), "inactive rows were written"
        if act_t.any():
            parity.check_outputs(o[act_t][None], o_ref[act_t][None], f"{name} step {t}")
        ended = act_t & (fill_before == w.period - 1)
        if ended.any():
            nc, ns = read()
            pre = np.stack([ref.last_pre[i] for i in np.nonzero(ended)[0]])
            parity.check_encoded(nc[ended], ns[ended], ref.codes[ended], ref.scales[ended], pre,
                                 f"{name} step {t} encode")
            ref.codes[ended], ref.scales[ended] = nc[ended], ns[ended]
            encodes += int(ended.sum())
        else:
            nc, _ = read()
            np.testing.assert_array_equal(nc, ref.codes)   # mid-period: codes untouched
    # flush ends every partial period
    partial = ref.fill > 0
    st.flush_steps()
    ref.flush()
    nc, ns = read()
    if partial.any():
        pre = np.stack([ref.last_pre[i] for i in np.nonzero(partial)[0]])
        parity.check_encoded(nc[partial], ns[partial], ref.codes[partial], ref.scales[partial],
                             pre, f"{name} flush")
    np.testing.assert_array_equal(nc[~partial], ref.codes[~partial])
    assert encodes > 0 and partial.any()
    s = st.stats()
    assert s["bytes_step_buffer"] == n * ((w.period - 1) * ((w.dk + w.dv) * 2 + 8) + 4)
    st.free()


def test_step_and_period_calls_are_exclusive():
    from linear_attn_decode_pace_amd import pace, runtime
    w = inputs.ragged("step-excl", 222, B=2, H=2, period=4, steps=4)
    say("[case] step / period exclusivity")
    bits = inputs.head_bits(w, 0)
    per = runtime.State(w, bits, pace.PACE_INIT_ZERO)
    stp = runtime.State(w, bits, pace.PACE_INIT_ZERO, flags=pace.PACE_STEP_BUFFER)
    tok = runtime.DeviceTokens(inputs.tokens(w, 0, inputs.SEG_DECODE, 0, 1))
    out = runtime.out_buffer(w, 1)
    with pytest.raises(pace.PaceError) as e:
        per.step(tok, out)
    assert e.value.status == pace.PACE_EINVAL
    with pytest.raises(pace.PaceError) as e:
        stp.decode(tok, out)
    assert e.value.status == pace.PACE_EINVAL
    with pytest.raises(pace.PaceError):
        pace.pace_flush_steps(per.handle)
    per.free()
    stp.free()


ADAPT_CASES = [
    ("adapt-k8", dict(B=3, H=5, n_int8=2, n_outliers=8, period=8, steps=40), 1.0, False),   # fused
    ("adapt-k8-mask", dict(B=3, H=5, n_int8=2, n_outliers=8, period=8, steps=40), 2.5, True),
    ("adapt-d64", dict(B=4, H=4, dk=64, dv=64, n_int8=1, period=8, steps=32), 1.0, False),
    ("adapt-f32", dict(B=2, H=3, n_int8=1, dtype=inputs.DT_F32, period=6, steps=30), 1.0, True),  # per-column
    ("adapt-dv80", dict(B=3, H=3, dv=80, n_int8=1, n_outliers=4, period=6, steps=24), 1.0, True),  # per-column
]


@pytest.mark.parametrize("name,kw,tau,masked", ADAPT_CASES)
def test_adaptive_period_against_buffered_oracle(name, kw, tau, masked):
    # adaptive period (PACE_ADAPTIVE): every step's close decision, outputs,
    # encodes and the per-state (A, R) against the oracle; a decision may
    # differ only where the oracle's A sits within 1e-4 of tau R, and then the
    # oracle follows the GPU
    import torch
    from linear_attn_decode_pace_amd import pace, runtime
    w = inputs.ragged(name, 230, **kw)
    seed = 0
    say(f"[case] adaptive period {name} tau={tau}")
    n = w.B * w.H
    idx = np.arange(n)
    bits = inputs.head_bits(w, seed)
    bits_t = np.tile(bits, w.B).astype(np.int64)
    st = runtime.State(w, bits, pace.PACE_INIT_F32, runtime.warmup_state(w, seed),
                       flags=pace.PACE_STEP_BUFFER | pace.PACE_ADAPTIVE, adapt_tau=tau)

    def read():
        c, s = st.read_codes()
        f, ar = st.read_step()
        return (c.reshape(n, w.dk, w.dv).cpu().numpy(), s.reshape(n, w.dv).cpu().numpy(),
                f.reshape(n).cpu().numpy(), ar.reshape(n, 2).cpu().numpy().astype(np.float64))

    codes, scales, fill, ar = read()
    ref = buffered.Buffered(codes, scales, bits_t, w.period, tau=tau)
    np.testing.assert_allclose(ar[:, 1], ref.R, rtol=1e-5)
    assert np.all(fill == 0) and np.all(ar[:, 0] == 0)
    rng = np.random.default_rng(6)
    lengths, near = [], 0
    for t in range(w.steps):
        act = rng.uniform(size=w.B) < 0.7 if masked else np.ones(w.B, dtype=bool)
        if t < 2:
            act[:] = True
        act_t = np.repeat(act, w.H)
        expect = np.array([ref.closes(i) for i in range(n)])
        marg = np.array([abs(ref.margin(i)) if ref.tau * ref.R[i] > 0 else np.inf for i in range(n)])
        fill_before = ref.fill
        tok = inputs.tokens(w, seed, inputs.SEG_DECODE, t, t + 1)
        out = runtime.out_buffer(w, 1).fill_(np.nan)
        st.step(runtime.DeviceTokens(tok), out, torch.as_tensor(act.astype(np.uint8), device="cuda"))
        nc, ns, nfill, nar = read()
        closed = act_t & (nfill == 0)
        bad = act_t & (closed != expect) & (marg >= 1e-4)
        assert not bad.any(), f"{name} step {t}: close decisions differ at {np.nonzero(bad)[0]}"
        near += int((act_t & (closed != expect)).sum())
        q, k, v, a, b = [x[0] for x in tok_tiles(tok, idx, w.H)]
        o_ref = ref.step(q, k, v, a, b, act_t, decide=closed)
        o = out.reshape(n, w.dv).cpu().numpy()
        assert np.all(np.isnan(o[~act_t]))
        if act_t.any():
            parity.check_outputs(o[act_t][None], o_ref[act_t][None], f"{name} step {t}")
        np.testing.assert_array_equal(nfill, ref.fill)
        if closed.any():
            lengths += (fill_before[closed] + 1).tolist()
            pre = np.stack([ref.last_pre[i] for i in np.nonzero(closed)[0]])
            parity.check_encoded(nc[closed], ns[closed], ref.codes[closed], ref.scales[closed], pre,
                                 f"{name} step {t} encode")
            ref.codes[closed], ref.scales[closed] = nc[closed], ns[closed]
            for i in np.nonzero(closed)[0]:
                ref.R[i] = ref._norm(i)
        np.testing.assert_array_equal(nc, ref.codes)
        np.testing.assert_allclose(nar[:, 1], ref.R, rtol=1e-5)
        np.testing.assert_allclose(nar[:, 0], ref.A, rtol=1e-4, atol=1e-6 * ref.R.max())
    say(f"[case] {name}: period lengths {np.bincount(lengths).tolist()}, {near} decisions on the threshold")
    assert len(set(lengths)) > 1   # the period really adapts
    partial = ref.fill > 0
    st.flush_steps()
    ref.flush()
    nc, ns, nfill, nar = read()
    assert np.all(nfill == 0) and np.all(nar[:, 0] == 0)
    if partial.any():
        pre = np.stack([ref.last_pre[i] for i in np.nonzero(partial)[0]])
        parity.check_encoded(nc[partial], ns[partial], ref.codes[partial], ref.scales[partial], pre,
                             f"{name} flush")
    # R is the norm of what the GPU stored (tie flips of the flush included)
    np.testing.assert_allclose(nar[:, 1], np.linalg.norm(quant.decode(nc, ns), axis=(1, 2)), rtol=1e-5)
    st.free()
