"""The C ABI library: it loads, exports what include/pace.h declares, and
rejects bad arguments before touching the device (no GPU needed)."""
import ctypes
import os
import re

import pytest

from linear_attn_decode_pace_amd import pace

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "pace.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pace_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(pace.LIB, n), n
    assert sorted(pace.EXPORTED) == names


def test_abi_version():
    assert pace.pace_abi_version() == 3


def _cfg(**kw):
    c = dict(batch=2, heads=2, d_k=128, d_v=128, period=8, in_dtype=pace.PACE_DTYPE_BF16,
             head_bits=[4, 8])
    c.update(kw)
    return c


def _alloc_status(init_kind=pace.PACE_INIT_ZERO, init=None, flags=0, **kw):
    c = _cfg(**kw)
    hb = (ctypes.c_uint8 * max(1, len(c["head_bits"])))(*c["head_bits"])
    cfg = pace.pace_config(c["batch"], c["heads"], c["d_k"], c["d_v"], c["period"], c["in_dtype"],
                           ctypes.cast(hb, ctypes.POINTER(ctypes.c_uint8)), flags,
                           c.get("adapt_tau", 0.0), c.get("fp8_window", 0))
    out = ctypes.c_void_p()
    return pace.LIB.pace_state_alloc(ctypes.byref(cfg), init_kind, init, None, ctypes.byref(out))


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), pace.PACE_EINVAL),
    (dict(heads=0, head_bits=[]), pace.PACE_EINVAL),
    (dict(d_k=96), pace.PACE_EUNSUPPORTED),
    (dict(d_v=100), pace.PACE_EUNSUPPORTED),
    (dict(d_v=512), pace.PACE_EUNSUPPORTED),
    (dict(period=0), pace.PACE_EUNSUPPORTED),
    (dict(period=65), pace.PACE_EUNSUPPORTED),
    (dict(in_dtype=7), pace.PACE_EINVAL),
    (dict(head_bits=[4, 6]), pace.PACE_EINVAL),
])
def test_alloc_rejects_bad_config(kw, status):
    assert _alloc_status(**kw) == status
    assert pace.pace_last_error() != ""


def test_alloc_rejects_bad_flags():
    assert _alloc_status(flags=16) == pace.PACE_EINVAL
    for bad in (0, 65):
        assert _alloc_status(flags=pace.PACE_FP8_WINDOW, fp8_window=bad) == pace.PACE_EINVAL
    assert _alloc_status(flags=pace.PACE_FP8_WINDOW | pace.PACE_STEP_BUFFER, fp8_window=8) == pace.PACE_EINVAL
    assert _alloc_status(flags=pace.PACE_ADAPTIVE, adapt_tau=0.5) == pace.PACE_EINVAL   # needs steps
    both = pace.PACE_ADAPTIVE | pace.PACE_STEP_BUFFER
    for tau in (0.0, -1.0, float("inf"), float("nan")):
        assert _alloc_status(flags=both, adapt_tau=tau) == pace.PACE_EINVAL
    many = pace.PACE_STATS_MAX_HEADS + 1
    assert _alloc_status(flags=pace.PACE_STATS_ERR, heads=many, head_bits=[4] * many) == pace.PACE_EINVAL
    assert "PACE_STATS_ERR" in pace.pace_last_error()


def test_stats_struct_matches_header():
    # the binding's pace_stats mirrors the C struct: same fields, same size
    src = open(os.path.join(ROOT, "include", "pace.h")).read()
    body = re.search(r"typedef struct pace_stats \{(.*?)\} pace_stats;", src, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"\b([a-z0-9_]+)(?:\[[A-Z_]+\])?;", body)
    assert names == [n for n, _ in pace.pace_stats._fields_]
    # sizes and offsets as the C compiler lays the struct out
    import subprocess
    import tempfile
    fields = [n for n, _ in pace.pace_stats._fields_]
    prog = "#include <stddef.h>\n#include <stdio.h>\n#include \"pace.h\"\nint main(void) {\n"
    prog += '    printf("%zu\\n", sizeof(pace_stats));\n'
    prog += "".join(f'    printf("%zu\\n", offsetof(pace_stats, {n}));\n' for n in fields)
    prog += "    return 0;\n}\n"
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "layout.c"), os.path.join(d, "layout")
        open(src, "w").write(prog)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        got = [int(x) for x in subprocess.run([exe], check=True, capture_output=True,
                                              text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(pace.pace_stats)
    assert got[1:] == [getattr(pace.pace_stats, n).offset for n in fields]


def test_alloc_rejects_bad_init():
    assert _alloc_status(init_kind=9) == pace.PACE_EINVAL
    assert _alloc_status(init_kind=pace.PACE_INIT_F32, init=None) == pace.PACE_EINVAL
    assert _alloc_status(init_kind=pace.PACE_INIT_F32, init=0x1004) == pace.PACE_EINVAL  # misaligned
    assert _alloc_status(init_kind=pace.PACE_INIT_ZERO, init=0x1000) == pace.PACE_EINVAL


def test_null_arguments():
    assert pace.LIB.pace_state_alloc(None, 0, None, None, None) == pace.PACE_EINVAL
    assert pace.LIB.pace_decode_period(None, 1, 16, 16, 16, 16, 16, 16, None) == pace.PACE_EINVAL
    assert pace.LIB.pace_read_state(None, 0, 16, 16, None) == pace.PACE_EINVAL
    assert pace.LIB.pace_quant_stats(None, None, None) == pace.PACE_EINVAL
    assert pace.LIB.pace_quant_stats_static(None, None, None) == pace.PACE_EINVAL
    assert pace.LIB.pace_raw_bytes(None, None) == pace.PACE_EINVAL
    assert pace.LIB.pace_decode_step(None, 16, 16, 16, 16, 16, None, 16, None) == pace.PACE_EINVAL
    assert pace.LIB.pace_flush_steps(None, None) == pace.PACE_EINVAL
    assert pace.LIB.pace_prefill_encode(None, 1, 16, 16, 16, 16, 16, None, None) == pace.PACE_EINVAL
    assert pace.LIB.pace_state_free(None) == pace.PACE_OK


def test_prefill_rejects_bad_arguments():
    f = pace.LIB.pace_prefill_f32
    good = (16, 32, 48, 64, 80)
    assert f(1, 1, 128, 128, 1, 9, *good, 96, None, None) == pace.PACE_EINVAL
    assert f(1, 1, 128, 128, 0, 1, *good, 96, None, None) == pace.PACE_EINVAL
    assert f(1, 1, 96, 128, 1, 1, *good, 96, None, None) == pace.PACE_EUNSUPPORTED
    assert f(1, 1, 128, 128, 1, 1, 17, 32, 48, 64, 80, 96, None, None) == pace.PACE_EINVAL
    assert f(1, 1, 128, 128, 1, 1, *good, None, None, None) == pace.PACE_EINVAL
    assert f(1, 1, 128, 128, 1, 1, *good, 100, None, None) == pace.PACE_EINVAL


def test_binding_raises_with_message():
    with pytest.raises(pace.PaceError) as e:
        pace.pace_state_alloc(1, 1, 96, 128, 8, pace.PACE_DTYPE_BF16, [4], stream=0)
    assert e.value.status == pace.PACE_EUNSUPPORTED and "d_k" in e.value.message


def test_stream_copy_rejects_bad_arguments():
    f = pace.LIB.pace_stream_copy
    assert f(None, 16, 32, None) == pace.PACE_EINVAL
    assert f(16, None, 32, None) == pace.PACE_EINVAL
    assert f(24, 16, 32, None) == pace.PACE_EINVAL   # misaligned dst
    assert f(16, 40, 32, None) == pace.PACE_EINVAL   # misaligned src
    assert f(16, 32, 40, None) == pace.PACE_EINVAL   # not a multiple of 16
    assert "multiple of 16" in pace.pace_last_error()


def _gpu_present() -> bool:
    import torch
    return torch.cuda.device_count() > 0   # counts devices without initialising them


def test_valid_alloc_without_a_device_is_edevice():
    # every argument is valid, so the call reaches the HIP runtime, which has
    # no device here: PACE_EDEVICE with the runtime's message, no handle
    if _gpu_present():
        pytest.skip("a GPU is present: a valid alloc succeeds")
    hb = (ctypes.c_uint8 * 2)(4, 8)
    cfg = pace.pace_config(2, 2, 128, 128, 8, pace.PACE_DTYPE_BF16,
                           ctypes.cast(hb, ctypes.POINTER(ctypes.c_uint8)), 0, 0.0, 0)
    out = ctypes.c_void_p()
    assert pace.LIB.pace_state_alloc(ctypes.byref(cfg), pace.PACE_INIT_ZERO, None, None,
                                     ctypes.byref(out)) == pace.PACE_EDEVICE
    assert out.value is None
    assert pace.pace_last_error() != ""
    # the same holds for the stateless entry points once their arguments pass
    assert pace.LIB.pace_stream_copy(16, 32, 64, None) == pace.PACE_EDEVICE
    assert pace.LIB.pace_prefill_f32(1, 1, 128, 128, 1, 1, 16, 32, 48, 64, 80, 96, None,
                                     None) == pace.PACE_EDEVICE
