"""Prefill hand-off (pace_prefill_encode) on the GPU against the oracle: a
prompt of n_tok tokens applied in float32 to the stored state and encoded
once, i.e. oracle.pace.period over the whole prompt."""
import numpy as np
import pytest

from linear_attn_decode_pace_amd import inputs
from oracle import quant
from oracle import pace as opace
from tests import parity
from tests.gpu_cases import say, tok_tiles

pytestmark = pytest.mark.gpu


def _run(w, seed, n_tok, warm, sample=None, outputs=True, tok_hook=None):
    import torch
    from linear_attn_decode_pace_amd import pace, runtime
    n = w.B * w.H
    idx = np.arange(n) if sample is None else np.asarray(sample)
    bits = inputs.head_bits(w, seed)
    bits_t = np.tile(bits, w.B)[idx].astype(np.int64)
    if warm:
        st = runtime.State(w, bits, pace.PACE_INIT_F32, runtime.warmup_state(w, seed))
    else:
        st = runtime.State(w, bits, pace.PACE_INIT_ZERO)
    tix = torch.as_tensor(idx, device="cuda")

    def read():
        c, s = st.read_codes()
        return (c.reshape(n, w.dk, w.dv)[tix].cpu().numpy(),
                s.reshape(n, w.dv)[tix].cpu().numpy())

    c0, s0 = read()
    tok = inputs.tokens(w, seed, inputs.SEG_PROMPT, 0, n_tok)
    if tok_hook is not None:
        tok = tok_hook(tok)
    out = runtime.out_buffer(w, n_tok) if outputs else None
    st.prefill(runtime.DeviceTokens(tok), out)
    c1, s1 = read()
    O, rc, rs, Mpre = opace.period(c0, s0, bits_t, *tok_tiles(tok, idx, w.H))
    what = f"{w.name} prefill {n_tok} tokens"
    rep = parity.check_encoded(c1, s1, rc, rs, Mpre, what)
    m = None
    if outputs:
        o = out.reshape(n_tok, n, w.dv)[:, tix].cpu().numpy()
        m = parity.check_outputs(o, O, what)
    st.free()
    say(f"[case] {what}: output rel err {m}, flips {rep.flips}")
    return rep


@pytest.mark.parametrize("name,kw,n_tok,warm", [
    ("pf-mixed", dict(B=2, H=3, n_int8=1, n_outliers=8), 100, False),   # 3 chunks of 32 + 4 tokens
    ("pf-warm", dict(B=3, H=5, n_int8=2, n_outliers=8), 37, True),      # from a warm stored state
    ("pf-d64", dict(B=4, H=4, dk=64, dv=64, n_int8=1), 50, False),
    ("pf-one", dict(B=2, H=2, n_int8=1), 1, True),
    ("pf-16", dict(B=2, H=3, n_int8=1), 16, False),                      # one half chunk
    ("pf-32", dict(B=2, H=3, n_int8=1), 32, True),                       # one whole chunk
    ("pf-two", dict(B=3, H=2, n_int8=1), 40, True),                      # two chunks: one per producer
    ("pf-three", dict(B=2, H=3, n_int8=1), 65, False),                   # odd chunk count, 1-token tail
    ("pf-five-d64", dict(B=2, H=3, dk=64, dv=64, n_int8=1), 150, True),  # 5 chunks, 22-token tail
    ("pf-f32", dict(B=2, H=3, n_int8=1, dtype=inputs.DT_F32), 40, False),  # per-column kernel
])
def test_prefill_encode(name, kw, n_tok, warm):
    w = inputs.ragged(name, 240, prompt=n_tok, warmup=0 if not warm else 32, **kw)
    _run(w, 0, n_tok, warm)


@pytest.mark.parametrize("value", [1e-5, 0.0])
def test_prefill_vanishing_decay(value):
    # every token of the even sequences decays by `value`: inside a chunk the
    # gate products underflow (1e-5) or are zero, so each chunk's state is
    # built from its own last tokens only
    import dataclasses
    w = inputs.ragged("pf-vanish", 242, B=4, H=3, n_int8=1, prompt=70, warmup=32)

    def hook(tok):
        a = tok.alpha.copy()
        a[:, 0::2] = np.float32(value)
        return dataclasses.replace(tok, alpha=a)

    _run(w, 0, 70, True, tok_hook=hook)


def test_prefill_encode_4096_tokens_sampled():
    # the prompt workload's per-tile shape (32 heads, 8 at 8 bits, 4096-token
    # prompts) on two sequences, checked on sampled tiles of both widths
    w = inputs.PREFILL.replace(B=2)
    bits = inputs.head_bits(w, 0)
    pick = sorted({0, 1, 31, 32, 63} | {int(h) for h in np.nonzero(bits == 8)[0][:3]}
                  | {32 + int(h) for h in np.nonzero(bits == 4)[0][-3:]})
    _run(w, 0, 4096, False, sample=np.array(pick))


def test_prefill_full_batch_sampled():
    # the prompt workload at its full size, in the launch bench.py times (512
    # sequences x 32 heads, one 4096-token prompt, fused encode): the prompt
    # is 64 distinct generated tokens repeated to 4096 on the device (bench.py
    # repeats 256), checked on sampled tiles of both widths
    import torch
    from linear_attn_decode_pace_amd import pace, runtime
    w = inputs.PREFILL
    T, D = 4096, 64
    n = w.B * w.H
    bits = inputs.head_bits(w, 0)
    say("[case] prefill-b512 full batch: generating 64 prompt tokens")
    tok = inputs.tokens(w, 0, inputs.SEG_PROMPT, 0, D)
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
    h8 = [int(h) for h in np.nonzero(bits == 8)[0][:2]]
    h4 = [int(h) for h in np.nonzero(bits == 4)[0][[0, -1]]]
    pairs = [(b, h) for b in (0, 255, 511) for h in h8 + h4]
    idx = np.array([b * w.H + h for b, h in pairs])
    tix = torch.as_tensor(idx, device="cuda")
    st = runtime.State(w, bits, pace.PACE_INIT_ZERO)
    out = runtime.out_buffer(w, T)
    st.prefill(big, out)
    torch.cuda.synchronize()
    c, s = st.read_codes()
    c1 = c.reshape(n, w.dk, w.dv)[tix].cpu().numpy()
    s1 = s.reshape(n, w.dv)[tix].cpu().numpy()
    o = out.reshape(T, n, w.dv)[:, tix].cpu().numpy()
    st.free()
    del big, out
    sel = tok.select([b for b, _ in pairs], [h for _, h in pairs])
    q, k, v, al, be = [np.tile(sel.f64(nm)[:, :, 0], (T // D,) + (1,) * (sel.f64(nm).ndim - 2))
                       for nm in ("q", "k", "v", "alpha", "beta")]
    bits_t = np.array([bits[h] for _, h in pairs], dtype=np.int64)
    zc = np.zeros((len(pairs), w.dk, w.dv), dtype=np.int64)
    zs = np.zeros((len(pairs), w.dv), dtype=np.float32)
    O, rc, rs, Mpre = opace.period(zc, zs, bits_t, q, k, v, al, be)
    what = f"prefill-b512 full batch, {T} tokens, {len(pairs)} sampled tiles"
    rep = parity.check_encoded(c1, s1, rc, rs, Mpre, what)
    m = parity.check_outputs(o, O, what)
    say(f"[case] {what}: output rel err {m}, flips {rep.flips}")


def test_prefill_encode_matches_float_prefill_then_encode():
    # the same prompt through pace_prefill_f32 + PACE_INIT_F32: both keep the
    # state in float32, so the stored states agree up to rounding ties
    import torch
    from linear_attn_decode_pace_amd import pace, runtime
    w = inputs.ragged("pf-cross", 241, B=2, H=4, n_int8=1, prompt=64, warmup=0)
    say("[case] prefill encode vs float prefill + encode")
    bits = inputs.head_bits(w, 0)
    tok = runtime.DeviceTokens(inputs.tokens(w, 0, inputs.SEG_PROMPT, 0, 64))
    a = runtime.State(w, bits, pace.PACE_INIT_ZERO)
    a.prefill(tok)
    M = torch.zeros((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    runtime.prefill(w, tok, M)
    b = runtime.State(w, bits, pace.PACE_INIT_F32, M)
    da, db = a.read_dequant(), b.read_dequant()
    rel = (torch.linalg.vector_norm(da - db) / torch.linalg.vector_norm(db)).item()
    assert rel < 2e-3, rel
    ca, _ = a.read_codes()
    cb, _ = b.read_codes()
    assert (ca != cb).float().mean().item() < 1e-3
    a.free()
    b.free()
