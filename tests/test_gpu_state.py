"""State handling on the GPU: checkpoint/resume, determinism, reads, stats, prefill."""
import numpy as np
import pytest

from linear_attn_decode_pace_amd import inputs
from oracle import gdn, quant
from oracle import pace as opace
from tests import parity
from tests.gpu_cases import say, tok_tiles

pytestmark = pytest.mark.gpu

W = inputs.ragged("state-mixed", 201, B=3, H=4, n_int8=1, n_outliers=8, steps=24)


def _state(w, seed, kind=None):
    from linear_attn_decode_pace_amd import pace, runtime
    bits = inputs.head_bits(w, seed)
    if kind is None:
        return runtime.State(w, bits, pace.PACE_INIT_F32, runtime.warmup_state(w, seed)), bits
    return runtime.State(w, bits, kind), bits


def _decode(st, w, seed, p):
    from linear_attn_decode_pace_amd import runtime
    tok = inputs.decode_period(w, seed, p)
    out = runtime.out_buffer(w, tok.T)
    st.decode(runtime.DeviceTokens(tok), out)
    return out


def test_raw_resume_is_bitwise():
    import torch
    from linear_attn_decode_pace_amd import pace, runtime
    say("[case] raw resume")
    a, bits = _state(W, 0)
    _decode(a, W, 0, 0)
    _decode(a, W, 0, 1)
    raw = a.read_raw()
    b = runtime.State(W, bits, pace.PACE_INIT_RAW, raw)
    assert torch.equal(b.read_raw(), raw)
    oa = _decode(a, W, 0, 2)
    ob = _decode(b, W, 0, 2)
    assert torch.equal(oa, ob)
    assert torch.equal(a.read_raw(), b.read_raw())


def test_two_runs_are_bitwise_equal():
    import torch
    say("[case] determinism")
    outs, raws = [], []
    for _ in range(2):
        st, _ = _state(W, 1)
        o = [_decode(st, W, 1, p) for p in range(3)]
        outs.append(torch.cat(o))
        raws.append(st.read_raw())
        st.free()
    assert torch.equal(outs[0], outs[1]) and torch.equal(raws[0], raws[1])


def test_read_dequant_is_codes_times_scales():
    import torch
    st, _ = _state(W, 2)
    _decode(st, W, 2, 0)
    c, s = st.read_codes()
    m = st.read_dequant()
    ref = c.float() * s[:, :, None, :]
    assert torch.equal(m, ref)


def test_raw_layout_holds_the_codes():
    # the raw image is [4-bit pool | 8-bit pool | scales]; its scales part equals the read scales
    import torch
    st, bits = _state(W, 3)
    raw = st.read_raw()
    _, s = st.read_codes()
    n_sc = W.B * W.H * W.dv * 4
    assert torch.equal(raw[-n_sc:].view(torch.float32).reshape(s.shape), s)
    n4 = int((bits == 4).sum())
    n8 = int((bits == 8).sum())
    assert raw.numel() == W.B * (n4 * W.dk * W.dv // 2 + n8 * W.dk * W.dv) + n_sc


def test_stats_closed_forms():
    from linear_attn_decode_pace_amd import pace
    w = inputs.MIXED.replace(B=8)
    st, bits = _state(w, 4)
    s = st.stats()
    d = w.dk
    assert s["heads4"] == 12 and s["heads8"] == 4
    assert s["bytes_codes4"] == w.B * 12 * d * d // 2
    assert s["bytes_codes8"] == w.B * 4 * d * d
    assert s["bytes_scales"] == w.B * w.H * d * 4
    assert s["bytes_total"] == s["bytes_codes4"] + s["bytes_codes8"] + s["bytes_scales"]
    assert s["bytes_fp16_equiv"] == w.B * w.H * d * d * 2
    ratio = s["bytes_total"] / s["bytes_int8_equiv"]
    assert abs(ratio - 1344 / 2112) < 1e-12          # about two thirds of all-8-bit
    assert s["zero_columns"] == 0 and s["periods"] == 0
    _decode(st, w, 4, 0)
    s = st.stats()
    assert s["periods"] == 1 and s["tokens"] == w.period
    st.free()
    z, _ = _state(w, 4, pace.PACE_INIT_ZERO)
    assert z.stats()["zero_columns"] == w.B * w.H * w.dv


def test_zero_state_decode():
    from linear_attn_decode_pace_amd import pace
    w = W
    st, bits = _state(w, 5, pace.PACE_INIT_ZERO)
    n = w.B * w.H
    bits_t = np.tile(bits, w.B).astype(np.int64)
    codes = np.zeros((n, w.dk, w.dv), np.int16)
    scales = np.zeros((n, w.dv), np.float32)
    for p in range(2):
        out = _decode(st, w, 5, p).reshape(w.period, n, w.dv).cpu().numpy()
        tok = inputs.decode_period(w, 5, p)
        q, k, v, a, b = tok_tiles(tok, np.arange(n), w.H)
        O, c2, s2, Mpre = opace.period(codes, scales, bits_t, q, k, v, a, b)
        parity.check_outputs(out, O, f"zero-init period {p}")
        c, s = st.read_codes()
        c = c.reshape(n, w.dk, w.dv).cpu().numpy()
        s = s.reshape(n, w.dv).cpu().numpy()
        parity.check_encoded(c, s, c2, s2, Mpre, f"zero-init period {p}")
        codes, scales = c, s


def test_prefill_outputs_and_state():
    import torch
    from linear_attn_decode_pace_amd import runtime
    w = inputs.ragged("prefill-small", 202, B=2, H=3, steps=8)
    tok = inputs.tokens(w, 0, inputs.SEG_PROMPT, 0, 40)
    M = torch.zeros((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    out = runtime.out_buffer(w, tok.T)
    runtime.prefill(w, runtime.DeviceTokens(tok), M, out)
    n = w.B * w.H
    q, k, v, a, b = tok_tiles(tok, np.arange(n), w.H)
    Mr, Or = gdn.run(np.zeros((n, w.dk, w.dv)), q, k, v, a, b)
    assert parity.rel_per_tile(M.reshape(n, w.dk, w.dv).cpu().numpy(), Mr, 0).max() <= 1e-5
    assert parity.rel_per_tile(out.reshape(tok.T, n, w.dv).cpu().numpy(), Or, 1).max() <= 1e-5


def test_enomem_for_absurd_batch():
    from linear_attn_decode_pace_amd import pace
    with pytest.raises(pace.PaceError) as e:
        pace.pace_state_alloc(1 << 26, 16, 128, 128, 8, pace.PACE_DTYPE_BF16, [4] * 16)
    assert e.value.status == pace.PACE_ENOMEM


def test_decode_rejects_too_many_tokens():
    from linear_attn_decode_pace_amd import pace, runtime
    st, _ = _state(W, 6)
    tok = runtime.DeviceTokens(inputs.tokens(W, 6, inputs.SEG_DECODE, 0, W.period + 1))
    out = runtime.out_buffer(W, tok.T)
    with pytest.raises(pace.PaceError) as e:
        st.decode(tok, out)
    assert e.value.status == pace.PACE_EINVAL


def _head_sums(per_tile, w):
    return per_tile.reshape(w.B, w.H).sum(axis=0)


@pytest.mark.parametrize("name,kw,n_tok", [
    ("err-k8", dict(B=3, H=5, n_int8=2, n_outliers=8), 8),          # 8-token fused kernel
    ("err-k12", dict(B=3, H=5, n_int8=2, period=16), 12),            # 16-token fused kernel
    ("err-f32", dict(B=2, H=3, n_int8=1, dtype=inputs.DT_F32), 8),   # per-column kernel
    ("err-d64", dict(B=4, H=4, dk=64, dv=64, n_int8=1), 8),
])
def test_error_statistics(name, kw, n_tok):
    # per-head sum (M - c s)^2 and sum M^2 of the state each encode quantized:
    # the initial encode of the warm state, then the period-end encode
    import torch
    from linear_attn_decode_pace_amd import pace, runtime
    w = inputs.ragged(name, 210, **kw)
    seed = 3
    say(f"[case] error statistics {name}")
    bits = inputs.head_bits(w, seed)
    bits_t = np.tile(bits, w.B)
    n = w.B * w.H
    M0 = runtime.warmup_state(w, seed)
    st = runtime.State(w, bits, pace.PACE_INIT_F32, M0, flags=pace.PACE_STATS_ERR)
    s = st.stats()
    assert s["err_tracked"] == 1
    M0g = M0.reshape(n, w.dk, w.dv).cpu().numpy().astype(np.float64)
    e, r = quant.roundtrip_error(M0g, bits_t)
    np.testing.assert_allclose(s["err_sq"], _head_sums(e, w), rtol=1e-4)
    np.testing.assert_allclose(s["ref_sq"], _head_sums(r, w), rtol=1e-5)

    codes, scales = st.read_codes()
    codes = codes.reshape(n, w.dk, w.dv).cpu().numpy()
    scales = scales.reshape(n, w.dv).cpu().numpy()
    tok = inputs.tokens(w, seed, inputs.SEG_DECODE, 0, n_tok)
    out = runtime.out_buffer(w, n_tok)
    st.decode(runtime.DeviceTokens(tok), out)
    torch.cuda.synchronize()
    _, _, _, Mpre = opace.period(codes, scales, bits_t, *tok_tiles(tok, np.arange(n), w.H))
    e, r = quant.roundtrip_error(Mpre, bits_t)
    s = st.stats()
    np.testing.assert_allclose(s["err_sq"], _head_sums(e, w), rtol=1e-3)
    np.testing.assert_allclose(s["ref_sq"], _head_sums(r, w), rtol=1e-4)
    st.free()


def test_error_statistics_off_and_zero_init():
    from linear_attn_decode_pace_amd import pace, runtime
    say("[case] error statistics without the flag / zero init")
    st, _ = _state(W, 0)
    s = st.stats()
    assert s["err_tracked"] == 0 and not any(s["err_sq"]) and not any(s["ref_sq"])
    st.free()
    z = runtime.State(W, inputs.head_bits(W, 0), pace.PACE_INIT_ZERO, flags=pace.PACE_STATS_ERR)
    s = z.stats()
    assert s["err_tracked"] == 1 and len(s["err_sq"]) == W.H
    assert not any(s["err_sq"]) and not any(s["ref_sq"])
    z.free()


@pytest.mark.parametrize("period,dk", [(8, 128), (16, 128), (8, 64), (16, 64)])
def test_every_code_value_decodes(period, dk):
    # A raw image whose code bytes are random (nibbles -7..7, bytes -127..127:
    # every code a stored state can hold, each column full of +-qmax, which an
    # encode only writes at its absmax entry).  The per-column reader and the
    # fused decode kernels must agree on every value: read_codes against the
    # bytes (as multisets, independent of the pool layout), then one period
    # against the oracle started from the codes read.
    import torch
    from linear_attn_decode_pace_amd import pace, runtime
    w = inputs.ragged(f"code-range-k{period}-d{dk}", 210, B=3, H=4, dk=dk, dv=dk, n_int8=2,
                      period=period, steps=period)
    say(f"[case] every code value: period {period}, d {dk}")
    st, bits = _state(w, 4)
    raw = st.read_raw()
    st.free()
    n4 = int((bits == 4).sum()) * w.B * dk * dk // 2
    n8 = int((bits == 8).sum()) * w.B * dk * dk
    rng = np.random.default_rng(11 + period + dk)
    b4 = rng.integers(0, 256, n4, dtype=np.uint8)
    b4 = np.where((b4 & 0x0F) == 0x08, b4 & 0xF0, b4)       # no nibble -8
    b4 = np.where((b4 & 0xF0) == 0x80, b4 & 0x0F, b4)
    b8 = rng.integers(0, 256, n8, dtype=np.uint8)
    b8 = np.where(b8 == 0x80, 0, b8).astype(np.uint8)         # no byte -128
    img = raw.clone()
    img[:n4 + n8] = torch.as_tensor(np.concatenate([b4, b8]), device=img.device)
    st = runtime.State(w, bits, pace.PACE_INIT_RAW, img)
    c, s = st.read_codes()
    n = w.B * w.H
    codes = c.reshape(n, dk, dk).cpu().numpy().astype(np.int64)
    scales = s.reshape(n, dk).cpu().numpy()
    bits_t = np.tile(bits, w.B).astype(np.int64)

    def signed4(x):
        x = x.astype(np.int64)
        return np.where(x >= 8, x - 16, x)
    want4 = np.bincount(np.concatenate([signed4(b4 & 0x0F), signed4(b4 >> 4)]) + 8, minlength=16)
    want8 = np.bincount(b8.view(np.int8).astype(np.int64) + 128, minlength=256)
    got4 = np.bincount(codes[bits_t == 4].ravel() + 8, minlength=16)
    got8 = np.bincount(codes[bits_t == 8].ravel() + 128, minlength=256)
    assert np.array_equal(got4, want4) and np.array_equal(got8, want8)
    assert got4[1] > 0 and got4[15] > 0 and got8[1] > 0 and got8[255] > 0  # -7, 7, -127, 127 present

    tok = inputs.decode_period(w, 4, 0)
    out = runtime.out_buffer(w, tok.T)
    st.decode(runtime.DeviceTokens(tok), out)
    o = out.reshape(tok.T, n, dk).cpu().numpy()
    nc, ns = st.read_codes()
    nc = nc.reshape(n, dk, dk).cpu().numpy()
    ns = ns.reshape(n, dk).cpu().numpy()
    q, k, v, a, b = tok_tiles(tok, np.arange(n), w.H)
    O, c2, s2, Mpre = opace.period(codes, scales, bits_t, q, k, v, a, b)
    m = parity.check_outputs(o, O, f"code range k={period} d={dk}")
    rep = parity.check_encoded(nc, ns, c2, s2, Mpre, f"code range k={period} d={dk}")
    say(f"[case] every code value: output rel err {m:.2e}, scale rel err {rep.max_scale:.2e}, "
        f"flips {rep.flips}/{rep.entries}")
    st.free()
