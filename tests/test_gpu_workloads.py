"""The measured workloads at their full sizes, in the launch configuration the
benchmark times, checked against the oracle on sampled tiles.

Every GPU launch covers the whole batch; the oracle replays and free-runs the
sampled (sequence, head) tiles one by one.  Samples always include the first
and last sequence and tiles of both bit widths.
"""
import numpy as np
import pytest

from linear_attn_decode_pace_amd import inputs
from oracle import gdn
from tests.gpu_cases import default_calls, run_case, say

pytestmark = pytest.mark.gpu

WORKERS = 16


def _sample(w, seed, n, rng_seed=0):
    bits = inputs.head_bits(w, seed)
    rng = np.random.default_rng(rng_seed)
    tiles = w.B * w.H
    pick = set(rng.choice(tiles, size=n, replace=False).tolist())
    pick |= {0, w.H - 1, tiles - w.H, tiles - 1}
    for width in (4, 8):
        hs = np.nonzero(bits == width)[0]
        if hs.size:
            pick |= {int(hs[0]), int((w.B - 1) * w.H + hs[-1])}
    return np.array(sorted(pick))


def test_headline_full_batch_sampled():
    # 4096 sequences x 16 heads (12 at 4 bits, 4 at 8 bits), period 8: the
    # benchmark's launch; three periods checked on 64+ sampled tiles
    w = inputs.HEADLINE
    run_case(w, 0, default_calls(w, 3), sample=_sample(w, 0, 64), workers=WORKERS)


def test_headline_steps_equal_period_calls():
    # the per-step form (one token per call, tokens buffered on the device)
    # at the headline's full size, in the launch the benchmark times for it
    # (one tile per workgroup, 65,536 tiles): a period of steps gives bitwise
    # the outputs and the stored state of one period call, which the sampled
    # oracle check above pins; mid-period steps leave the stored state alone
    import torch

    from linear_attn_decode_pace_amd import pace, runtime

    w = inputs.HEADLINE.replace(warmup=8)
    seed = 0
    bits = inputs.head_bits(w, seed)
    wtok = inputs.concat(inputs.iter_tokens(
        w, seed, inputs.SEG_WARMUP, [(t, t + 1) for t in range(w.warmup)], WORKERS))
    M0 = runtime.warmup_state(w, seed, tok=wtok)
    per = runtime.State(w, bits, pace.PACE_INIT_F32, M0)
    stp = runtime.State(w, bits, pace.PACE_INIT_F32, M0, flags=pace.PACE_STEP_BUFFER)
    del M0
    C = w.period
    for p in range(2):
        say(f"[case] headline steps vs period call, period {p}")
        tok = inputs.concat(inputs.iter_tokens(
            w, seed, inputs.SEG_DECODE, [(t, t + 1) for t in range(p * C, (p + 1) * C)], WORKERS))
        dt = runtime.DeviceTokens(tok)
        out_p = runtime.out_buffer(w, C)
        per.decode(dt, out_p)
        raw0 = stp.read_raw()
        for t in range(C):
            out_s = runtime.out_buffer(w, 1)
            stp.step(dt.slice(t, t + 1), out_s)
            assert torch.equal(out_s[0], out_p[t]), f"period {p} token {t}"
            if t < C - 1:
                assert torch.equal(stp.read_raw(), raw0), f"period {p} token {t} wrote"
        assert torch.equal(stp.read_raw(), per.read_raw()), f"state after period {p}"
        del raw0, out_p, dt
    per.free()
    stp.free()


def test_headline_fp8_window_sampled():
    # the FP8 write window at the headline's full size in the launch its
    # bench times (8 writes kept per state, 4096 x 16 states): ten steps, so
    # the window fills and then merges its oldest write into the stored
    # history twice; before each step the window oracle is rebuilt for 32+
    # sampled tiles from what the GPU stores, then both take the step
    import torch

    from linear_attn_decode_pace_amd import pace, runtime
    from tests import parity
    from tests.gpu_cases import tok_tiles
    from tests.test_gpu_window import _oracle_from

    w = inputs.HEADLINE.replace(warmup=8)
    S, seed = 8, 0
    n = w.B * w.H
    idx = _sample(w, seed, 32)
    idx_t = torch.as_tensor(idx, device="cuda")
    bits = np.tile(inputs.head_bits(w, seed), w.B).astype(np.int64)[idx]
    wtok = inputs.concat(inputs.iter_tokens(
        w, seed, inputs.SEG_WARMUP, [(t, t + 1) for t in range(w.warmup)], WORKERS))
    M0 = runtime.warmup_state(w, seed, tok=wtok)
    st = runtime.State(w, inputs.head_bits(w, seed), pace.PACE_INIT_F32, M0,
                       flags=pace.PACE_FP8_WINDOW, fp8_window=S)
    del M0

    def sampled_state():
        c, sc = st.read_codes()
        wc, wf = st.read_window()
        cnt, meta = st.read_step()
        pick = lambda x, *shape: x.reshape(n, *shape)[idx_t].cpu().numpy()
        return (pick(c, w.dk, w.dv), pick(sc, w.dv), pick(wc, S, w.dk + w.dv), pick(wf, S, 3),
                pick(cnt), pick(meta, 2))

    merges = 0
    for t in range(S + 2):
        say(f"[case] headline fp8 window S={S}, step {t}")
        before = sampled_state()
        ref = _oracle_from(before, bits, S, w.dk)
        tok = inputs.tokens(w, seed, inputs.SEG_DECODE, t, t + 1)
        out = runtime.out_buffer(w, 1)
        st.step(runtime.DeviceTokens(tok), out)
        q, k, v, a, b = [x[0] for x in tok_tiles(tok, idx, w.H)]
        o_ref = ref.step(q, k, v, a, b)
        o = out.reshape(n, w.dv)[idx_t].cpu().numpy()
        parity.check_outputs(o[None], o_ref[None], f"headline window step {t}")
        c, sc, wc, wf, cnt, meta = sampled_state()
        np.testing.assert_array_equal(cnt, [len(ref.win[i]) for i in range(len(idx))])
        np.testing.assert_allclose(meta[:, 0], ref.lam, rtol=1e-6)
        merged = before[4] == S
        if merged.any():
            merges += int(merged.sum())
            pre = np.stack([ref.last_pre[i] for i in np.nonzero(merged)[0]])
            parity.check_encoded(c[merged], sc[merged], ref.codes[merged], ref.scales[merged], pre,
                                 f"headline window step {t} merge", lattice_ties=True)
        else:
            np.testing.assert_array_equal(c, before[0])   # no merge: history untouched
    assert merges == 2 * len(idx)
    st.free()


@pytest.mark.parametrize("tau", [1.0, 2.5])
def test_headline_adaptive_period_sampled(tau):
    # the adaptive period at the headline's full size in the launch its bench
    # times (per-step calls, one tile per workgroup, maximum period 8):
    # twelve steps of the whole batch; on 32+ sampled tiles every close
    # decision, output, encode and (A, R) against the buffered oracle, which
    # follows the GPU only where its A sits within 1e-4 of tau R
    import torch

    from linear_attn_decode_pace_amd import pace, runtime
    from oracle import buffered
    from tests import parity
    from tests.gpu_cases import tok_tiles

    w = inputs.HEADLINE.replace(warmup=8)
    seed = 0
    n = w.B * w.H
    idx = _sample(w, seed, 32)
    m = len(idx)
    idx_t = torch.as_tensor(idx, device="cuda")
    bits = inputs.head_bits(w, seed)
    wtok = inputs.concat(inputs.iter_tokens(
        w, seed, inputs.SEG_WARMUP, [(t, t + 1) for t in range(w.warmup)], WORKERS))
    M0 = runtime.warmup_state(w, seed, tok=wtok)
    st = runtime.State(w, bits, pace.PACE_INIT_F32, M0,
                       flags=pace.PACE_STEP_BUFFER | pace.PACE_ADAPTIVE, adapt_tau=tau)
    del M0

    def read():
        c, sc = st.read_codes()
        fl, ar = st.read_step()
        pick = lambda x, *shape: x.reshape(n, *shape)[idx_t].cpu().numpy()
        return pick(c, w.dk, w.dv), pick(sc, w.dv), pick(fl), pick(ar, 2).astype(np.float64)

    codes, scales, fill, ar = read()
    ref = buffered.Buffered(codes, scales, np.tile(bits, w.B).astype(np.int64)[idx], w.period, tau=tau)
    np.testing.assert_allclose(ar[:, 1], ref.R, rtol=1e-5)
    closes = 0
    for t in range(12):
        say(f"[case] headline adaptive period tau={tau}, step {t}")
        expect = np.array([ref.closes(i) for i in range(m)])
        marg = np.array([abs(ref.margin(i)) if ref.tau * ref.R[i] > 0 else np.inf for i in range(m)])
        tok = inputs.tokens(w, seed, inputs.SEG_DECODE, t, t + 1)
        out = runtime.out_buffer(w, 1)
        st.step(runtime.DeviceTokens(tok), out)
        nc, ns, nfill, nar = read()
        closed = nfill == 0
        bad = (closed != expect) & (marg >= 1e-4)
        assert not bad.any(), f"step {t}: close decisions differ at tiles {idx[bad]}"
        q, k, v, a, b = [x[0] for x in tok_tiles(tok, idx, w.H)]
        o_ref = ref.step(q, k, v, a, b, np.ones(m, dtype=bool), decide=closed)
        o = out.reshape(n, w.dv)[idx_t].cpu().numpy()
        parity.check_outputs(o[None], o_ref[None], f"adaptive step {t}")
        np.testing.assert_array_equal(nfill, ref.fill)
        if closed.any():
            closes += int(closed.sum())
            pre = np.stack([ref.last_pre[i] for i in np.nonzero(closed)[0]])
            parity.check_encoded(nc[closed], ns[closed], ref.codes[closed], ref.scales[closed], pre,
                                 f"adaptive step {t} encode")
            ref.codes[closed], ref.scales[closed] = nc[closed], ns[closed]
            for i in np.nonzero(closed)[0]:
                ref.R[i] = ref._norm(i)
        np.testing.assert_array_equal(nc, ref.codes)
        np.testing.assert_allclose(nar[:, 1], ref.R, rtol=1e-5)
        np.testing.assert_allclose(nar[:, 0], ref.A, rtol=1e-4, atol=1e-6 * ref.R.max())
    assert closes > 0
    st.free()


def test_mixed_b1024_whole_run_sampled():
    # 1024 sequences, all 512 decode steps (64 periods), outlier channels
    w = inputs.MIXED
    r = run_case(w, 0, default_calls(w), sample=_sample(w, 0, 24), workers=WORKERS)
    assert r["calls"] == 64


@pytest.mark.parametrize("period", [1, 2, 4, 8, 16])
def test_sweep_b256_whole_run_sampled(period):
    # 256 sequences, 256 decode steps at each period length
    w = inputs.SWEEP.replace(period=period)
    run_case(w, 0, default_calls(w), sample=_sample(w, 0, 24), workers=WORKERS,
             label=f"sweep-b256-k{period}")


def test_prompt_decode_full_batch_sampled():
    # the prompt workload's decode at its full size, in the launch the
    # benchmark times (512 sequences x 32 heads, 8 at 8 bits, period 16: the
    # 16-token chunk kernel), from a 32-token warm state; two periods checked
    # on 32+ sampled tiles
    w = inputs.PREFILL.replace(warmup=32)
    run_case(w, 0, default_calls(w, 2), sample=_sample(w, 0, 32), workers=WORKERS,
             label="prefill-b512-decode")


def test_prompt_handoff_reduced_batch():
    # 4096-token prompts through the library's float32 prefill into the
    # quantized state, then decode at period 16 with 8 of 32 heads at 8 bits;
    # the batch is reduced from 512 to 8 prompts (input volume), every other
    # size is the workload's own
    import torch

    from linear_attn_decode_pace_amd import runtime

    w = inputs.PREFILL.replace(B=8, steps=64)
    seed = 0
    idx = _sample(w, seed, 16)
    M = torch.zeros((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    Mr = np.zeros((len(idx), w.dk, w.dv))
    blk = 256
    ranges = [(t, min(w.prompt, t + blk)) for t in range(0, w.prompt, blk)]
    b, h = idx // w.H, idx % w.H
    for i, tok in enumerate(inputs.iter_tokens(w, seed, inputs.SEG_PROMPT, ranges, WORKERS)):
        runtime.prefill(w, runtime.DeviceTokens(tok), M)
        arr = [tok.f64(x)[:, b, h] for x in ("q", "k", "v", "alpha", "beta")]
        Mr, _ = gdn.run(Mr, *arr)
        if i % 4 == 0:
            say(f"[case] prompt tokens up to {ranges[i][1]}")
    # hand-off state: float32 chunk-free prefill vs float64, 2e-3 relative L2
    run_case(w, seed, default_calls(w), sample=idx, workers=WORKERS, M0_gpu=M, M0_ref=Mr,
             label="prefill-b8-handoff", warm_rel=2e-3)


def test_prompt_handoff_full_batch_then_decode():
    # the prompt workload end to end at its full size: 512 prompts x 32 heads
    # (8 at 8 bits) of 4096 tokens through pace_prefill_encode into the
    # quantized state (the prompt is 64 distinct generated tokens repeated on
    # the device), then two period-16 decode calls from that stored state;
    # the hand-off and every decode transition checked on 32+ sampled tiles
    import torch

    from linear_attn_decode_pace_amd import pace, runtime
    from oracle import pace as opace
    from tests import parity
    from tests.gpu_cases import tok_tiles

    w = inputs.PREFILL
    T, D, seed = w.prompt, 64, 0
    n = w.B * w.H
    bits = inputs.head_bits(w, seed)
    idx = _sample(w, seed, 32)
    bits_t = np.tile(bits, w.B)[idx].astype(np.int64)
    tix = torch.as_tensor(idx, device="cuda")
    say(f"[case] prefill-b512 hand-off + decode: {T}-token prompts ({D} distinct), {len(idx)} tiles")
    tok = inputs.concat(inputs.iter_tokens(
        w, seed, inputs.SEG_PROMPT, [(t, t + inputs.TB) for t in range(0, D, inputs.TB)], WORKERS))
    small = runtime.DeviceTokens(tok)
    big = runtime.DeviceTokens.__new__(runtime.DeviceTokens)
    for name in ("q", "k", "v", "alpha", "beta"):
        x = getattr(small, name)
        y = torch.empty((T,) + tuple(x.shape[1:]), dtype=x.dtype, device="cuda")
        for t0 in range(0, T, D):
            y[t0:t0 + D].copy_(x)
        setattr(big, name, y)
    big.T = T
    del small
    st = runtime.State(w, bits, pace.PACE_INIT_ZERO)
    st.prefill(big)
    del big

    def read():
        c, s = st.read_codes()
        return (c.reshape(n, w.dk, w.dv)[tix].cpu().numpy(), s.reshape(n, w.dv)[tix].cpu().numpy())

    codes, scales = read()
    q, k, v, a, b = [np.tile(x, (T // D,) + (1,) * (x.ndim - 1)) for x in tok_tiles(tok, idx, w.H)]
    zc = np.zeros((len(idx), w.dk, w.dv), dtype=np.int64)
    zs = np.zeros((len(idx), w.dv), dtype=np.float32)
    _, rc, rs, Mpre = opace.period(zc, zs, bits_t, q, k, v, a, b)
    del q, k, v, a, b
    rep = parity.check_encoded(codes, scales, rc, rs, Mpre, f"prefill-b512 hand-off of {T} tokens")
    fc, fs = rc, rs   # free-running oracle from its own hand-off
    diverged = np.any(codes.astype(np.int16) != fc, axis=(1, 2))
    calls = default_calls(w, 2)
    for ci, dtok in enumerate(inputs.iter_tokens(w, seed, inputs.SEG_DECODE, calls, WORKERS)):
        out = runtime.out_buffer(w, dtok.T)
        st.decode(runtime.DeviceTokens(dtok), out)
        o = out.reshape(dtok.T, n, w.dv)[:, tix].cpu().numpy()
        nc, ns = read()
        args = tok_tiles(dtok, idx, w.H)
        what = f"prefill-b512 decode call {ci} after the hand-off"
        O, c2, s2, M2 = opace.period(codes, scales, bits_t, *args)
        parity.check_outputs(o, O, what)
        rep = rep.merge(parity.check_encoded(nc, ns, c2, s2, M2, what))
        Of, fc, fs, Mf = opace.period(fc, fs, bits_t, *args)
        live = ~diverged
        if live.any():
            parity.check_outputs(o[:, live], Of[:, live], what + " (free-running)")
        diverged |= np.any(nc.astype(np.int16) != fc, axis=(1, 2))
        codes, scales = nc, ns
    st.free()
    say(f"[case] prefill-b512 hand-off + decode: ok, {rep.flips} tie flips, "
        f"{int(diverged.sum())} tiles diverged by a tie")
