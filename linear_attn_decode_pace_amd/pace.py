"""Thin ctypes binding of libpace.so (include/pace.h).

Argument marshalling only: every step of the decode path runs in the HIP
library.  Functions carry the C names.  Tensor arguments may be torch tensors
(their data_ptr() is passed) or integer device addresses; ``stream`` defaults
to torch's current stream on the current device.

The library must have been built (``python -m linear_attn_decode_pace_amd.build``);
there is no fallback: a missing library raises at import of this module.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# PACE_LIBRARY may name another build of the same ABI (e.g. the host-sanitizer
# build the CPU tests make); by default the in-tree libpace.so is loaded
LIB_PATH = os.environ.get("PACE_LIBRARY") or os.path.join(_HERE, "libpace.so")

PACE_OK = 0
PACE_EINVAL = -1
PACE_ENOMEM = -2
PACE_EUNSUPPORTED = -3
PACE_EDEVICE = -4

PACE_DTYPE_F32 = 0
PACE_DTYPE_BF16 = 1

PACE_INIT_ZERO = 0
PACE_INIT_F32 = 1
PACE_INIT_RAW = 2

PACE_READ_CODES = 0
PACE_READ_DEQUANT = 1
PACE_READ_RAW = 2
PACE_READ_STEP = 3
PACE_READ_WINDOW = 4

PACE_STATS_ERR = 0x1
PACE_STEP_BUFFER = 0x2
PACE_ADAPTIVE = 0x4
PACE_FP8_WINDOW = 0x8
PACE_STATS_MAX_HEADS = 256

EXPORTED = ("pace_abi_version", "pace_last_error", "pace_state_alloc", "pace_state_free",
            "pace_state_config", "pace_raw_bytes", "pace_decode_period", "pace_read_state",
            "pace_quant_stats", "pace_prefill_f32", "pace_decode_step", "pace_flush_steps",
            "pace_prefill_encode", "pace_stream_copy", "pace_quant_stats_static")


class PaceError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pace status {status}: {message}")
        self.status = status
        self.message = message


class pace_config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("period", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("head_bits", ctypes.POINTER(ctypes.c_uint8)), ("flags", ctypes.c_uint32),
                ("adapt_tau", ctypes.c_float), ("fp8_window", ctypes.c_int32)]


class pace_stats(ctypes.Structure):
    _fields_ = [("bytes_codes4", ctypes.c_uint64), ("bytes_codes8", ctypes.c_uint64),
                ("bytes_scales", ctypes.c_uint64), ("bytes_total", ctypes.c_uint64),
                ("bytes_fp16_equiv", ctypes.c_uint64), ("bytes_int8_equiv", ctypes.c_uint64),
                ("heads4", ctypes.c_int32), ("heads8", ctypes.c_int32),
                ("periods", ctypes.c_uint64), ("tokens", ctypes.c_uint64),
                ("zero_columns", ctypes.c_uint64), ("bytes_step_buffer", ctypes.c_uint64),
                ("err_tracked", ctypes.c_int32),
                ("err_sq", ctypes.c_double * PACE_STATS_MAX_HEADS),
                ("ref_sq", ctypes.c_double * PACE_STATS_MAX_HEADS)]

    def as_dict(self, heads: int = PACE_STATS_MAX_HEADS):
        d = {name: getattr(self, name) for name, _ in self._fields_}
        d["err_sq"] = list(self.err_sq)[:heads]
        d["ref_sq"] = list(self.ref_sq)[:heads]
        return d


def _load():
    # torch first: its bundled HIP runtime carries the same soname as the one
    # libpace.so was linked against, so the loader binds libpace.so to it and
    # the process holds a single HIP runtime (two copies do not share devices).
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m linear_attn_decode_pace_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    sig = {
        "pace_abi_version": ([], ctypes.c_int),
        "pace_last_error": ([], ctypes.c_char_p),
        "pace_state_alloc": ([ctypes.POINTER(pace_config), ctypes.c_int, vp, vp,
                              ctypes.POINTER(vp)], ctypes.c_int),
        "pace_state_free": ([vp], ctypes.c_int),
        "pace_state_config": ([vp, ctypes.POINTER(pace_config)], ctypes.c_int),
        "pace_raw_bytes": ([vp, ctypes.POINTER(ctypes.c_uint64)], ctypes.c_int),
        "pace_decode_period": ([vp, i32, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "pace_read_state": ([vp, ctypes.c_int, vp, vp, vp], ctypes.c_int),
        "pace_quant_stats": ([vp, ctypes.POINTER(pace_stats), vp], ctypes.c_int),
        "pace_prefill_f32": ([i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp],
                             ctypes.c_int),
        "pace_decode_step": ([vp, vp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "pace_flush_steps": ([vp, vp], ctypes.c_int),
        "pace_prefill_encode": ([vp, i32, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
        "pace_stream_copy": ([vp, vp, ctypes.c_uint64, vp], ctypes.c_int),
        "pace_quant_stats_static": ([vp, ctypes.POINTER(pace_stats), vp], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


LIB = _load()


def pace_last_error() -> str:
    return LIB.pace_last_error().decode()


def pace_abi_version() -> int:
    return LIB.pace_abi_version()


def _check(status: int) -> None:
    if status != PACE_OK:
        raise PaceError(status, pace_last_error())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def pace_state_alloc(batch: int, heads: int, d_k: int, d_v: int, period: int, in_dtype: int,
                     head_bits: Sequence[int], init_kind: int = PACE_INIT_ZERO, init=None,
                     flags: int = 0, stream=None, adapt_tau: float = 0.0,
                     fp8_window: int = 0) -> int:
    """Allocate and initialise the pools; returns the opaque handle (an int)."""
    hb = (ctypes.c_uint8 * max(1, len(head_bits)))(*[int(b) for b in head_bits])
    cfg = pace_config(batch, heads, d_k, d_v, period, in_dtype,
                      ctypes.cast(hb, ctypes.POINTER(ctypes.c_uint8)), flags, adapt_tau,
                      fp8_window)
    out = ctypes.c_void_p()
    _check(LIB.pace_state_alloc(ctypes.byref(cfg), init_kind, _ptr(init), _stream(stream),
                                ctypes.byref(out)))
    return out.value


def pace_state_free(st: int) -> None:
    _check(LIB.pace_state_free(st))


def pace_state_config(st: int) -> dict:
    c = pace_config()
    _check(LIB.pace_state_config(st, ctypes.byref(c)))
    return {"batch": c.batch, "heads": c.heads, "d_k": c.d_k, "d_v": c.d_v,
            "period": c.period, "in_dtype": c.in_dtype,
            "head_bits": [c.head_bits[i] for i in range(c.heads)], "flags": c.flags,
            "adapt_tau": c.adapt_tau, "fp8_window": c.fp8_window}


def pace_raw_bytes(st: int) -> int:
    n = ctypes.c_uint64()
    _check(LIB.pace_raw_bytes(st, ctypes.byref(n)))
    return n.value


def pace_decode_period(st: int, n_tok: int, q, k, v, alpha, beta, out, stream=None) -> None:
    _check(LIB.pace_decode_period(st, n_tok, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                  _ptr(beta), _ptr(out), _stream(stream)))


def pace_decode_step(st: int, q, k, v, alpha, beta, out, active=None, stream=None) -> None:
    _check(LIB.pace_decode_step(st, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                _ptr(active), _ptr(out), _stream(stream)))


def pace_prefill_encode(st: int, n_tok: int, q, k, v, alpha, beta, out=None, stream=None) -> None:
    _check(LIB.pace_prefill_encode(st, n_tok, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                   _ptr(out), _stream(stream)))


def pace_stream_copy(dst, src, nbytes: int, stream=None) -> None:
    _check(LIB.pace_stream_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)))


def pace_flush_steps(st: int, stream=None) -> None:
    _check(LIB.pace_flush_steps(st, _stream(stream)))


def pace_read_state(st: int, what: int, dst, scales_dst=None, stream=None) -> None:
    _check(LIB.pace_read_state(st, what, _ptr(dst), _ptr(scales_dst), _stream(stream)))


def pace_quant_stats(st: int, stream=None) -> dict:
    s = pace_stats()
    _check(LIB.pace_quant_stats(st, ctypes.byref(s), _stream(stream)))
    return s.as_dict(pace_state_config(st)["heads"])


def pace_quant_stats_static(st: int, stream=None) -> dict:
    s = pace_stats()
    _check(LIB.pace_quant_stats_static(st, ctypes.byref(s), _stream(stream)))
    return s.as_dict(pace_state_config(st)["heads"])


def pace_prefill_f32(batch: int, heads: int, d_k: int, d_v: int, n_tok: int, in_dtype: int,
                     q, k, v, alpha, beta, state, out=None, stream=None) -> None:
    _check(LIB.pace_prefill_f32(batch, heads, d_k, d_v, n_tok, in_dtype, _ptr(q), _ptr(k),
                                _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(out),
                                _stream(stream)))
