"""The device-free host-library tests again, against the host code built with
AddressSanitizer and UndefinedBehaviorSanitizer (lib/libchunkattn_hostsan.so,
built next to the library by the package build).

They run in a child process with the compiler's ASan runtime preloaded (the
sanitized library does not link it) and the binding pointed at the sanitized
build; any sanitizer report ends that process with an error.  Covered: the
argument validation of every entry point, the host and device-free plans,
the C++ streaming-queue bookkeeping, status strings and error paths.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SANITIZED = os.path.join(ROOT, "chunked_spatio_temporal_amd", "lib", "libchunkattn_hostsan.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def asan_runtime():
    hits = sorted(glob.glob(os.path.join(ROCM, "lib", "llvm", "lib", "clang", "*", "lib",
                                         "linux", "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def test_host_library_under_address_and_ub_sanitizers():
    rt = asan_runtime()
    if not os.path.exists(SANITIZED) or rt is None:
        pytest.skip("sanitized host library or ASan runtime not available")
    env = dict(os.environ)
    env.update({
        "CHUNKATTN_LIBRARY": SANITIZED,
        "LD_PRELOAD": rt,
        # Python and the libraries it loads are not instrumented: their
        # allocations are not leak-checked
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    probe = ("import ctypes; from chunked_spatio_temporal_amd import chunkattn as ca; "
             "lib = ca.load_library(); "
             "assert ca.LIB_PATH.endswith('libchunkattn_hostsan.so'), ca.LIB_PATH; "
             "assert hasattr(ctypes.CDLL(None), '__asan_report_load8'); "
             "assert b'__ubsan_handle' in open(ca.LIB_PATH, 'rb').read(); print('sanitized ok')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and "sanitized ok" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", os.path.join("tests", "test_host_library.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
