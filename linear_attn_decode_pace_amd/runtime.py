"""Torch-side helpers around the C ABI: device buffers, a state wrapper, warm-up.

PyTorch is used only for device memory and streams; every step of the decode
path runs in libpace.so through ``pace``.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import inputs, pace


def dtype_code(w: inputs.Workload) -> int:
    return pace.PACE_DTYPE_BF16 if w.dtype == inputs.DT_BF16 else pace.PACE_DTYPE_F32


def _tensor(a: np.ndarray, bf16: bool, device) -> torch.Tensor:
    if bf16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device, non_blocking=False)


class DeviceTokens:
    """The five input tensors of a run of tokens, resident on the device."""

    def __init__(self, tok: inputs.Tokens, device="cuda"):
        bf16 = tok.dtype == inputs.DT_BF16
        self.q = _tensor(tok.q, bf16, device)
        self.k = _tensor(tok.k, bf16, device)
        self.v = _tensor(tok.v, bf16, device)
        self.alpha = _tensor(tok.alpha, False, device)
        self.beta = _tensor(tok.beta, False, device)
        self.T = tok.T

    def slice(self, t0: int, t1: int) -> "DeviceTokens":
        d = DeviceTokens.__new__(DeviceTokens)
        d.q, d.k, d.v = self.q[t0:t1], self.k[t0:t1], self.v[t0:t1]
        d.alpha, d.beta = self.alpha[t0:t1], self.beta[t0:t1]
        d.T = t1 - t0
        return d

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.q, self.k, self.v, self.alpha, self.beta))


class State:
    """Owns one pace_state handle (pools of B x H quantized states)."""

    def __init__(self, w: inputs.Workload, head_bits: Sequence[int],
                 init_kind: int = pace.PACE_INIT_ZERO, init: Optional[torch.Tensor] = None,
                 period: Optional[int] = None, stream=None, flags: int = 0,
                 adapt_tau: float = 0.0, fp8_window: int = 0):
        self.w = w
        self.head_bits = np.asarray(head_bits, dtype=np.uint8)
        self.period = w.period if period is None else period
        self.fp8_window = fp8_window
        self.handle = pace.pace_state_alloc(w.B, w.H, w.dk, w.dv, self.period, dtype_code(w),
                                            list(self.head_bits), init_kind, init, flags, stream,
                                            adapt_tau, fp8_window)

    def free(self):
        if self.handle:
            pace.pace_state_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass

    def decode(self, tok: DeviceTokens, out: torch.Tensor, stream=None):
        pace.pace_decode_period(self.handle, tok.T, tok.q, tok.k, tok.v, tok.alpha, tok.beta,
                                out, stream)

    def prefill(self, tok: DeviceTokens, out: Optional[torch.Tensor] = None, stream=None):
        """A prompt of tok.T tokens applied in float32 and encoded once."""
        pace.pace_prefill_encode(self.handle, tok.T, tok.q, tok.k, tok.v, tok.alpha, tok.beta,
                                 out, stream)

    def step(self, tok: DeviceTokens, out: torch.Tensor, active: Optional[torch.Tensor] = None,
             stream=None):
        """One decode step of a PACE_STEP_BUFFER handle: tok holds one token
        ([1, B, H, d]); active is a device uint8 [B] mask or None."""
        if tok.T != 1:
            raise ValueError("a step takes exactly one token")
        pace.pace_decode_step(self.handle, tok.q, tok.k, tok.v, tok.alpha, tok.beta, out,
                              active, stream)

    def flush_steps(self, stream=None):
        pace.pace_flush_steps(self.handle, stream)

    def read_step(self, stream=None):
        """Buffered tokens per state [B, H] (int32) and (A, R) [B, H, 2]."""
        w = self.w
        fill = torch.empty((w.B, w.H), dtype=torch.int32, device="cuda")
        ar = torch.empty((w.B, w.H, 2), dtype=torch.float32, device="cuda")
        pace.pace_read_state(self.handle, pace.PACE_READ_STEP, fill, ar, stream)
        return fill, ar

    def read_window(self, stream=None):
        """FP8 window of a PACE_FP8_WINDOW handle: codes [B, H, S, d_k + d_v]
        (uint8) and per slot (k scale, u scale, decay) [B, H, S, 3]."""
        w, S = self.w, self.fp8_window
        codes = torch.empty((w.B, w.H, S, w.dk + w.dv), dtype=torch.uint8, device="cuda")
        f = torch.empty((w.B, w.H, S, 3), dtype=torch.float32, device="cuda")
        pace.pace_read_state(self.handle, pace.PACE_READ_WINDOW, codes, f, stream)
        return codes, f

    def read_codes(self, stream=None):
        w = self.w
        codes = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.int8, device="cuda")
        scales = torch.empty((w.B, w.H, w.dv), dtype=torch.float32, device="cuda")
        pace.pace_read_state(self.handle, pace.PACE_READ_CODES, codes, scales, stream)
        return codes, scales

    def read_dequant(self, stream=None):
        w = self.w
        m = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
        pace.pace_read_state(self.handle, pace.PACE_READ_DEQUANT, m, None, stream)
        return m

    def read_raw(self, stream=None):
        n = pace.pace_raw_bytes(self.handle)
        raw = torch.empty(n, dtype=torch.uint8, device="cuda")
        pace.pace_read_state(self.handle, pace.PACE_READ_RAW, raw, None, stream)
        return raw

    def stats(self, stream=None) -> dict:
        return pace.pace_quant_stats(self.handle, stream)


def out_buffer(w: inputs.Workload, n_tok: int, device="cuda") -> torch.Tensor:
    return torch.empty((n_tok, w.B, w.H, w.dv), dtype=torch.float32, device=device)


def prefill(w: inputs.Workload, tok: DeviceTokens, state: torch.Tensor,
            out: Optional[torch.Tensor] = None, stream=None) -> None:
    pace.pace_prefill_f32(w.B, w.H, w.dk, w.dv, tok.T, dtype_code(w), tok.q, tok.k, tok.v,
                          tok.alpha, tok.beta, state, out, stream)


def warmup_state(w: inputs.Workload, seed: int, device="cuda",
                 tok: Optional[inputs.Tokens] = None) -> torch.Tensor:
    """float32 state after the workload's unquantized warm-up tokens from zero,
    computed by the library's prefill kernel (tok: the warm-up tokens, if
    already generated)."""
    M = torch.zeros((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=device)
    if w.warmup:
        if tok is None:
            tok = inputs.warmup_tokens(w, seed)
        prefill(w, DeviceTokens(tok, device), M)
    return M
