"""Launches too large for 32-bit per-token offsets: 16,384 sequences x 16
heads = 262,144 states at d = 128, where one token's inputs and outputs span
more than 2^31 bytes of a period's buffers.  The fused kernels index tokens
with 64-bit offsets (the prefill switches to its 64-bit instantiation), so
such batches run the same kernels as small ones.  Checked against the oracle
on sampled tiles that include the last sequences (the largest offsets)."""
import numpy as np
import pytest

from linear_attn_decode_pace_amd import inputs
from oracle import pace as opace
from tests import parity
from tests.gpu_cases import run_case, say, tok_tiles
from tests.test_gpu_workloads import _sample

pytestmark = pytest.mark.gpu

WORKERS = 16
B_LARGE = 16384

# the per-column kernel takes ~90 ms per 8-token period at this size and the
# fused one ~1.5 ms: a launch under this bound ran the fused kernel
FUSED_MS = 20.0


def _large(**kw):
    return inputs.HEADLINE.replace(name="mixed-b16384", B=B_LARGE, **kw)


def test_decode_large_batch_sampled():
    # two 8-token periods (8-token kernel) and one of 12 tokens (16-token
    # kernel; the handle's period is 16, so the 8-token calls are shorter
    # periods), mixed 4/8-bit heads with column outliers, 48+ sampled tiles
    w = _large(warmup=8, period=16)
    assert w.B * w.H >= 262144
    run_case(w, 0, [(0, 8), (8, 16), (16, 28)], sample=_sample(w, 0, 48), workers=WORKERS)


def test_decode_large_batch_runs_fused():
    import torch

    from linear_attn_decode_pace_amd import pace, runtime

    w = _large(warmup=0)
    st = runtime.State(w, inputs.head_bits(w, 0), pace.PACE_INIT_ZERO)
    tok = runtime.DeviceTokens(inputs.concat(inputs.iter_tokens(
        w, 0, inputs.SEG_DECODE, [(0, 8)], WORKERS)))
    out = runtime.out_buffer(w, 8)
    st.decode(tok, out)  # first launch loads the code object
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    st.decode(tok, out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    say(f"[case] {w.name}: 8-token period over {w.B * w.H} states in {ms:.2f} ms")
    st.free()
    assert ms < FUSED_MS, f"{ms:.1f} ms per period: the fused kernel did not run"


def test_prefill_large_batch_sampled():
    # a 40-token prompt (two 32-token chunks, one per producer) from a zero
    # state: the prefill's 64-bit instantiation
    import torch

    from linear_attn_decode_pace_amd import pace, runtime

    n_tok = 40
    w = _large(warmup=0, prompt=n_tok)
    seed = 0
    n = w.B * w.H
    idx = _sample(w, seed, 48)
    bits = inputs.head_bits(w, seed)
    bits_t = np.tile(bits, w.B)[idx].astype(np.int64)
    say(f"[case] {w.name} prefill {n_tok} tokens over {n} states")
    st = runtime.State(w, bits, pace.PACE_INIT_ZERO)
    tok = inputs.concat(inputs.iter_tokens(
        w, seed, inputs.SEG_PROMPT,
        [(t, min(n_tok, t + inputs.TB)) for t in range(0, n_tok, inputs.TB)], WORKERS))
    out = runtime.out_buffer(w, n_tok)
    st.prefill(runtime.DeviceTokens(tok), out)
    tix = torch.as_tensor(idx, device="cuda")
    c, s = st.read_codes()
    c1 = c.reshape(n, w.dk, w.dv)[tix].cpu().numpy()
    s1 = s.reshape(n, w.dv)[tix].cpu().numpy()
    o = out.reshape(n_tok, n, w.dv)[:, tix].cpu().numpy()
    st.free()
    z_c = np.zeros((len(idx), w.dk, w.dv), dtype=np.int16)
    z_s = np.zeros((len(idx), w.dv), dtype=np.float32)
    O, rc, rs, Mpre = opace.period(z_c, z_s, bits_t, *tok_tiles(tok, idx, w.H))
    what = f"{w.name} prefill {n_tok} tokens"
    rep = parity.check_encoded(c1, s1, rc, rs, Mpre, what)
    m = parity.check_outputs(o, O, what)
    say(f"[case] {what}: output rel err {m:.3g}, flips {rep.flips}")
