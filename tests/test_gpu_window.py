"""FP8 write window (PACE_FP8_WINDOW) on the GPU against oracle/window.py.

A column dominated by a merged FP8 write has its quotients at 7 (or 127)
times an E4M3 value over the largest, i.e. on exact half-integers, so a
merge's encode may flip every such tie (each flip still within the tie
tolerance); see parity.check_encoded(lattice_ties).

Transition validity, step by step: before every step the oracle is rebuilt
from what the GPU stores (the history's codes and scales, its decay, and the
window's E4M3 codes, scales and decays in ring order), then both take the
step.  Outputs must agree to float32 accuracy; the new write's E4M3 codes must
be equal except where the oracle's float32 quotient sits on a rounding
midpoint; a merge's history encode is checked like every other encode.
bf16 inputs at d_k = d_v = 64 or 128 run the fused wavefront-per-state kernel,
float32 inputs the per-column one.  Masked steps must leave the outputs and
every stored byte of inactive sequences untouched.
"""
import numpy as np
import pytest

from linear_attn_decode_pace_amd import inputs
from oracle import window
from tests import parity
from tests.gpu_cases import say, tok_tiles

pytestmark = pytest.mark.gpu

MID_TOL = 1e-4  # relative distance of a quotient to an E4M3 rounding midpoint


def _midpoint_distance(q: np.ndarray) -> np.ndarray:
    """Distance of each float32 quotient to the nearest E4M3 midpoint, in quanta."""
    a = np.abs(q.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    quantum = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - 3))
    x = a / quantum
    return np.abs(np.abs(x - np.floor(x)) - 0.5)


def _gpu_state(st, w, S):
    n = w.B * w.H
    c, s = st.read_codes()
    wc, wf = st.read_window()
    cnt, meta = st.read_step()
    return (c.reshape(n, w.dk, w.dv).cpu().numpy(), s.reshape(n, w.dv).cpu().numpy(),
            wc.reshape(n, S, w.dk + w.dv).cpu().numpy(), wf.reshape(n, S, 3).cpu().numpy(),
            cnt.reshape(n).cpu().numpy(), meta.reshape(n, 2).cpu().numpy())


def _oracle_from(gpu, bits, S, dk):
    c, s, wc, wf, cnt, meta = gpu
    ref = window.Window(c, s, bits, S)
    for i in range(c.shape[0]):
        ref.lam[i] = float(meta[i, 0])
        head = int(meta[i, 1])
        for e in range(int(cnt[i])):
            slot = (head + e) % S
            ref.win[i].append([wc[i, slot, :dk].copy(), np.float32(wf[i, slot, 0]),
                               wc[i, slot, dk:].copy(), np.float32(wf[i, slot, 1]),
                               float(wf[i, slot, 2])])
    return ref


CASES = [
    ("win-s4", dict(B=2, H=3, n_int8=1, n_outliers=8, steps=14), 4),
    ("win-s1", dict(B=2, H=2, n_int8=1, steps=6), 1),
    ("win-d64", dict(B=3, H=2, dk=64, dv=64, n_int8=1, steps=10), 3),
    ("win-f32", dict(B=2, H=2, n_int8=1, dtype=inputs.DT_F32, steps=8), 2),
    # more than 8 entries: the key dot products take two groups of lanes
    ("win-s12", dict(B=2, H=3, n_int8=1, steps=16), 12),
    # 256 states in 64 workgroups: two whole groups of the XCD order
    ("win-xcd", dict(B=16, H=16, dk=64, dv=64, n_int8=4, steps=5), 3),
    # d_v != d_k: the per-column window kernels
    ("win-dv80", dict(B=2, H=3, dv=80, n_int8=1, n_outliers=4, steps=8), 3),
    ("win-dv48", dict(B=2, H=2, dk=64, dv=48, n_int8=1, steps=6), 2),
]


@pytest.mark.parametrize("name,kw,S", CASES)
def test_window_steps_against_oracle(name, kw, S):
    _run(name, kw, S, masked=False)


@pytest.mark.parametrize("name,kw,S", [CASES[0], CASES[2], CASES[3], CASES[6]])
def test_window_masked_steps(name, kw, S):
    _run(name + "-mask", kw, S, masked=True)


@pytest.mark.parametrize("name,kw,S", [CASES[0], CASES[2]])
def test_window_tiny_columns(name, kw, S):
    # the even state columns start at 1e-37 of their values (scales near the
    # bottom of float32's normal range): a merge's lam alpha s then falls
    # below it, while the merged write keeps the new column normal
    _run(name + "-tiny", kw, S, masked=False, tiny_cols=True)


def _run(name, kw, S, masked, tiny_cols=False):
    import torch
    from linear_attn_decode_pace_amd import pace, runtime
    w = inputs.ragged(name, 250, **kw)
    seed = 0
    say(f"[case] fp8 window {name} S={S}")
    n = w.B * w.H
    idx = np.arange(n)
    bits = np.tile(inputs.head_bits(w, seed), w.B).astype(np.int64)
    M0 = runtime.warmup_state(w, seed)
    if tiny_cols:
        M0[..., 0::2] *= 1e-37
    st = runtime.State(w, inputs.head_bits(w, seed), pace.PACE_INIT_F32, M0,
                       flags=pace.PACE_FP8_WINDOW, fp8_window=S)
    rng = np.random.default_rng(11)
    flips = entries = merges = 0
    for t in range(w.steps):
        act = np.ones(w.B, bool)
        if masked and t >= 1:
            act = rng.uniform(size=w.B) < 0.6
        act_t = np.repeat(act, w.H)
        before = _gpu_state(st, w, S)
        ref = _oracle_from(before, bits, S, w.dk)
        cnt0, head0 = before[4], before[5][:, 1].astype(int)
        tok = inputs.tokens(w, seed, inputs.SEG_DECODE, t, t + 1)
        out = runtime.out_buffer(w, 1).fill_(np.nan)
        st.step(runtime.DeviceTokens(tok), out,
                torch.as_tensor(act.astype(np.uint8), device="cuda") if masked else None)
        q, k, v, a, b = [x[0] for x in tok_tiles(tok, idx, w.H)]
        o_ref = ref.step(q, k, v, a, b)
        o = out.reshape(n, w.dv).cpu().numpy()
        assert np.all(np.isnan(o[~act_t])), f"{name} step {t}: inactive rows were written"
        if act_t.any():
            parity.check_outputs(o[act_t][None], o_ref[act_t][None], f"{name} step {t}")
        after = _gpu_state(st, w, S)
        for x0, x1 in zip(before, after):
            np.testing.assert_array_equal(x1[~act_t], x0[~act_t], f"{name} step {t}: inactive state changed")
        c, s, wc, wf, cnt, meta = after
        for i in np.nonzero(act_t)[0]:
            slot = (head0[i] + cnt0[i]) % S
            kc, ks, uc, us, _ = ref.win[i][-1]
            assert np.array_equal(wc[i, slot, :w.dk], kc) and wf[i, slot, 0] == ks, f"{name} step {t} key"
            assert abs(wf[i, slot, 1] - us) <= 1e-6 * us, f"{name} step {t} u scale"
            diff = wc[i, slot, w.dk:] != uc
            if diff.any():
                # the oracle's quotients of the differing codes must sit on a midpoint
                M = _oracle_from(before, bits, S, w.dk).state(i)
                u = b[i] * (v[i] - a[i] * (k[i] @ M))
                qv = np.clip(np.asarray(u, np.float32) / np.float32(us), -448, 448)
                assert np.all(_midpoint_distance(qv[diff]) < MID_TOL), f"{name} step {t} u codes"
                flips += int(diff.sum())
            entries += w.dv
        np.testing.assert_array_equal(cnt[act_t], [len(ref.win[i]) for i in np.nonzero(act_t)[0]])
        np.testing.assert_allclose(meta[act_t, 0], ref.lam[act_t], rtol=1e-6)
        merged = (cnt0 == S) & act_t
        if merged.any():
            merges += int(merged.sum())
            pre = np.stack([ref.last_pre[i] for i in np.nonzero(merged)[0]])
            parity.check_encoded(c[merged], s[merged], ref.codes[merged], ref.scales[merged], pre,
                                 f"{name} step {t} merge", lattice_ties=True)
        # decays of the window, oldest first, against the oracle's
        for i in np.nonzero(act_t)[0]:
            head = int(meta[i, 1])
            got = [wf[i, (head + e) % S, 2] for e in range(int(cnt[i]))]
            np.testing.assert_allclose(got, [e_[4] for e_ in ref.win[i]], rtol=1e-6)
    assert merges > 0 or S >= w.steps
    assert flips <= 1e-3 * entries
    say(f"[case] {name}: {merges} merges, {flips} FP8 tie flips of {entries} codes")
    # flush: the whole window into the history
    before = _gpu_state(st, w, S)
    ref = _oracle_from(before, bits, S, w.dk)
    st.flush_steps()
    ref.flush()
    c, s, wc, wf, cnt, meta = _gpu_state(st, w, S)
    assert not cnt.any() and np.all(meta[:, 0] == 1.0)
    full = before[4] > 0
    pre = np.stack([ref.last_pre[i] for i in np.nonzero(full)[0]])
    parity.check_encoded(c[full], s[full], ref.codes[full], ref.scales[full], pre, f"{name} flush",
                         lattice_ties=True)
    s_ = st.stats()
    assert s_["bytes_step_buffer"] == n * (S * (w.dk + w.dv + 12) + 12)
    st.free()


@pytest.mark.parametrize("name,kw", [
    ("win-err", dict(B=3, H=5, n_int8=2, n_outliers=8)),                # fused kernel
    ("win-err-f32", dict(B=2, H=3, n_int8=1, dtype=inputs.DT_F32)),    # per-column kernel
])
def test_window_error_statistics(name, kw):
    # PACE_STATS_ERR on a window handle: a merge's encode reports, per head,
    # sum (H - c s)^2 and sum H^2 of the history it quantized
    from oracle import quant
    from linear_attn_decode_pace_amd import pace, runtime
    S = 3
    w = inputs.ragged(name, 251, **kw)
    seed = 2
    say(f"[case] window error statistics {name}")
    n = w.B * w.H
    bits = np.tile(inputs.head_bits(w, seed), w.B).astype(np.int64)
    st = runtime.State(w, inputs.head_bits(w, seed), pace.PACE_INIT_F32,
                       runtime.warmup_state(w, seed),
                       flags=pace.PACE_FP8_WINDOW | pace.PACE_STATS_ERR, fp8_window=S)
    for t in range(S):
        tok = inputs.tokens(w, seed, inputs.SEG_DECODE, t, t + 1)
        st.step(runtime.DeviceTokens(tok), runtime.out_buffer(w, 1))
    before = _gpu_state(st, w, S)
    assert np.all(before[4] == S)
    ref = _oracle_from(before, bits, S, w.dk)
    tok = inputs.tokens(w, seed, inputs.SEG_DECODE, S, S + 1)
    st.step(runtime.DeviceTokens(tok), runtime.out_buffer(w, 1))
    ref.step(*[x[0] for x in tok_tiles(tok, np.arange(n), w.H)])
    pre = np.stack(ref.last_pre)
    e, r = quant.roundtrip_error(pre, bits)
    s = st.stats()
    assert s["err_tracked"] == 1
    np.testing.assert_allclose(s["err_sq"], e.reshape(w.B, w.H).sum(axis=0), rtol=1e-3)
    np.testing.assert_allclose(s["ref_sq"], r.reshape(w.B, w.H).sum(axis=0), rtol=1e-4)
    st.free()
