"""Runner for GPU-vs-oracle decode cases, shared by the GPU tests."""
from __future__ import annotations

import sys
from typing import List, Optional, Sequence, Tuple

import numpy as np

from linear_attn_decode_pace_amd import inputs
from oracle import gdn, quant
from oracle import pace as opace
from tests import parity

WARM_REL = 1e-5  # float32 warm-up against float64, 32 tokens from zero


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def tok_tiles(tok: inputs.Tokens, idx: np.ndarray, H: int):
    """float64 [T, n, ...] arrays of the tiles idx (tile = b * H + h)."""
    b, h = idx // H, idx % H
    out = []
    for name in ("q", "k", "v", "alpha", "beta"):
        a = tok.f64(name)[:, b, h]
        out.append(a)
    return out


def default_calls(w: inputs.Workload, n_periods: Optional[int] = None) -> List[Tuple[int, int]]:
    n = w.periods if n_periods is None else n_periods
    return [(p * w.period, (p + 1) * w.period) for p in range(n)]


def run_case(w: inputs.Workload, seed: int, calls: Sequence[Tuple[int, int]],
             sample: Optional[np.ndarray] = None, head_bits=None,
             free_running: bool = True, label: str = "", workers: int = 1,
             M0_gpu=None, M0_ref=None, warm_rel: float = WARM_REL,
             tok_hook=None) -> dict:
    """Warm up, encode and decode on the GPU through the C ABI; check every
    step against the oracle on the tiles in ``sample`` (all tiles if None).
    tok_hook(call index, tokens) may replace each call's tokens (both sides
    then see the replaced ones)."""
    import torch

    from linear_attn_decode_pace_amd import pace, runtime

    label = label or w.name
    say(f"[case] {label}: B={w.B} H={w.H} d={w.dk}x{w.dv} period={w.period} dtype={w.dtype} "
        f"calls={len(calls)} seed={seed}")
    n = w.B * w.H
    idx = np.arange(n) if sample is None else np.asarray(sample)
    bits = inputs.head_bits(w, seed) if head_bits is None else np.asarray(head_bits, np.uint8)
    bits_t = np.tile(bits, w.B)[idx].astype(np.int64)

    # warm-up: GPU prefill kernel vs oracle recurrence, each from its own zero
    # state (or states handed in by the caller, e.g. after a long prompt)
    if M0_gpu is None:
        wtok = None
        if w.warmup:
            wtok = inputs.concat(inputs.iter_tokens(
                w, seed, inputs.SEG_WARMUP,
                [(t, min(w.warmup, t + inputs.TB)) for t in range(0, w.warmup, inputs.TB)], workers))
        M0_gpu = runtime.warmup_state(w, seed, tok=wtok)
        if w.warmup:
            wq, wk, wv, wa, wb = tok_tiles(wtok, idx, w.H)
            M0_ref = gdn.from_zero(w.dk, w.dv, wq, wk, wv, wa, wb)
    M0g = M0_gpu.reshape(n, w.dk, w.dv)[torch.as_tensor(idx, device="cuda")].cpu().numpy().astype(np.float64)
    if M0_ref is not None:
        M0r = M0_ref
        err = parity.rel_per_tile(M0g, M0r, 0).max()
        say(f"[case] {label}: starting-state rel err {err:.3g}")
        assert err <= warm_rel, f"{label}: starting-state rel err {err:.3g}"
    else:
        M0r = np.zeros_like(M0g)

    st = runtime.State(w, bits, pace.PACE_INIT_F32, M0_gpu)
    tix = torch.as_tensor(idx, device="cuda")

    def read():
        c, s = st.read_codes()
        c = c.reshape(n, w.dk, w.dv)[tix].cpu().numpy()
        s = s.reshape(n, w.dv)[tix].cpu().numpy()
        return c, s

    codes, scales = read()
    rc, rs = quant.encode(M0g, bits_t)
    rep = parity.check_encoded(codes, scales, rc, rs, M0g, f"{label} initial encode")
    # free-running oracle trajectory from its own warm-up
    fc, fs = quant.encode(M0r, bits_t)
    diverged = np.zeros(len(idx), dtype=bool)
    if free_running:
        diverged |= np.any(codes.astype(np.int16) != fc, axis=(1, 2))

    max_out = 0.0
    free_max_out = 0.0
    for ci, ((t0, t1), tok) in enumerate(zip(calls, inputs.iter_tokens(w, seed, inputs.SEG_DECODE,
                                                                       calls, workers))):
        if tok_hook is not None:
            tok = tok_hook(ci, tok)
        dt = runtime.DeviceTokens(tok)
        out = runtime.out_buffer(w, tok.T)
        st.decode(dt, out)
        o = out.reshape(tok.T, n, w.dv)[:, tix].cpu().numpy()
        nc, ns = read()
        q, k, v, a, b = tok_tiles(tok, idx, w.H)
        # transition validity: replay from the state the GPU stored
        O, c2, s2, Mpre = opace.period(codes, scales, bits_t, q, k, v, a, b)
        what = f"{label} call {ci} tokens [{t0},{t1})"
        max_out = max(max_out, parity.check_outputs(o, O, what))
        rep = rep.merge(parity.check_encoded(nc, ns, c2, s2, Mpre, what))
        # free-running comparison on tiles without an upstream tie flip
        if free_running:
            Of, fc, fs, Mf = opace.period(fc, fs, bits_t, q, k, v, a, b)
            live = ~diverged
            if live.any():
                free_max_out = max(free_max_out, parity.check_outputs(o[:, live], Of[:, live],
                                                                      what + " (free-running)"))
                parity.check_encoded(nc[live], ns[live], fc[live], fs[live], Mf[live],
                                     what + " (free-running)")
            diverged |= np.any(nc.astype(np.int16) != fc, axis=(1, 2))
        codes, scales = nc, ns
    st.free()
    res = dict(label=label, tiles=len(idx), calls=len(calls), flips=rep.flips,
               entries=rep.entries, max_out=max_out, free_max_out=free_max_out,
               max_scale=rep.max_scale, max_state_masked=rep.max_state_masked,
               diverged_tiles=int(diverged.sum()))
    say(f"[case] {label}: ok {res}")
    return res
