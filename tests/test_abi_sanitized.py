"""The C ABI layer (pace_abi.cpp) under the host AddressSanitizer and
UndefinedBehaviorSanitizer: a sanitizer build of the library runs the whole
CPU ABI suite (tests/test_abi_cpu.py: every argument check, the storage
struct layout, PACE_EDEVICE with no device) in a subprocess, and any
sanitizer report fails it.  Device code is built as usual; only the host
side of pace_abi.cpp is instrumented."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib", "llvm")
SAN_LIB = os.path.join(ROOT, "_build", "libpace_san.so")
# host-only instrumentation (each sanitizer flag applies to the host pass)
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _asan_runtime():
    hits = glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so"))
    return hits[0] if hits else None


def _build_sanitized():
    from linear_attn_decode_pace_amd import build as b
    b.build()  # the regular objects (device kernels) the sanitized library links
    obj = os.path.join(b.BUILD, "pace_abi_san.o")
    cmd = [b._hipcc(), "-x", "hip", *b.CFLAGS, *SAN_FLAGS, "-I", os.path.join(ROOT, "include"),
           "-c", os.path.join(b.CSRC, "pace_abi.cpp"), "-o", obj]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    objs = [obj] + [os.path.join(b.BUILD, os.path.splitext(s)[0] + ".o")
                    for s in b.SOURCES if s != "pace_abi.cpp"]
    link = [os.path.join(LLVM, "bin", "clang++"), "-shared", "-fPIC", "-shared-libsan",
            *SAN_FLAGS, "-o", SAN_LIB, *objs,
            "-L", os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib"), "-lamdhip64"]
    subprocess.run(link, check=True, capture_output=True, text=True)


def test_abi_suite_under_host_sanitizers():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime in this ROCm install")
    _build_sanitized()
    syms = subprocess.run(["nm", "-D", SAN_LIB], check=True, capture_output=True, text=True).stdout
    assert "__asan_report_load" in syms and "__ubsan_handle" in syms   # instrumented
    env = dict(os.environ)
    env.update(PACE_LIBRARY=SAN_LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    log = r.stdout + r.stderr
    # the suite ran against the sanitizer build, with the runtime loaded
    probe = subprocess.run([sys.executable, "-c",
                            "from linear_attn_decode_pace_amd import pace; "
                            "m = open('/proc/self/maps').read(); "
                            "print(pace.LIB_PATH, 'libpace_san.so' in m, 'libclang_rt.asan' in m)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.stdout.split() == [SAN_LIB, "True", "True"], probe.stdout + probe.stderr
    assert "AddressSanitizer" not in log and "runtime error:" not in log, log[-4000:]
    assert r.returncode == 0, log[-4000:]
    assert " passed" in r.stdout
