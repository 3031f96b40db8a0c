"""Builds the gfx950 HIP library lib/libchunkattn.so in-tree.

Run as ``python -m chunked_spatio_temporal_amd._build``; ``__graft_entry__.build()``
calls build().  Every build recompiles from source, in three steps:

1. the device code alone (gfx950 code object in an offload bundle), with the
   compiler kept from forming packed fp32 VALU instructions
   (``-target-feature -packed-fp32-ops``, a device-only feature);
2. the host code alone, with that device binary embedded and registered at
   load time (``-fcuda-include-gpubinary``, as the HIP driver does itself);
3. the shared library from the host object and the HIP runtime.

Next to it the same host code is built once more with AddressSanitizer and
UndefinedBehaviorSanitizer (host pass only, on the same device binary) into
lib/libchunkattn_hostsan.so, for the CPU tests of the host library under the
sanitizers (tests/test_host_sanitized.py).  Its sanitizer runtime is not
linked in: a process loads it with the compiler's ASan runtime preloaded.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libchunkattn.so")
SANITIZED_LIB = os.path.join(LIBDIR, "libchunkattn_hostsan.so")
SOURCE = os.path.join(CSRC, "chunkattn_api.hip")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.environ.get("HIP_CLANG", os.path.join(ROCM, "lib", "llvm", "bin", "clang++"))
ARCH = "gfx950"

COMMON = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-Wall",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE_ONLY = ["--cuda-device-only",
               # keep the compiler from forming packed fp32 VALU ops
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_ONLY = ["--cuda-host-only", "-fPIC"]
# host-side sanitizers (each flag for the host compilation only)
HOST_SANITIZE = ["-O1", "-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _host_library(fatbin, out, flags, verbose):
    obj = out + ".o.tmp"
    tmp = out + ".tmp"
    try:
        _run([CLANG, *COMMON, *HOST_ONLY, *flags, "-Xclang", "-fcuda-include-gpubinary",
              "-Xclang", fatbin, "-c", SOURCE, "-o", obj], verbose)
        _run([CLANG, "-shared", obj, "-o", tmp, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
              f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"], verbose)
        os.replace(tmp, out)
    finally:
        for p in (obj, tmp):
            if os.path.exists(p):
                os.remove(p)


def build(verbose: bool = False, extra=(), sanitized: bool = True) -> str:
    """Compiles the library (and, with `sanitized`, its host-sanitized twin);
    `extra` flags go to both the device and host steps."""
    os.makedirs(LIBDIR, exist_ok=True)
    fatbin = LIB + ".hipfb.tmp"
    try:
        _run([CLANG, *COMMON, *DEVICE_ONLY, *extra, SOURCE, "-o", fatbin], verbose)
        _host_library(fatbin, LIB, list(extra), verbose)
        if sanitized:
            _host_library(fatbin, SANITIZED_LIB, [*extra, *HOST_SANITIZE], verbose)
    finally:
        if os.path.exists(fatbin):
            os.remove(fatbin)
    return LIB


if __name__ == "__main__":
    extra = [a for a in sys.argv[1:] if a != "-v"]
    print(build(verbose="-v" in sys.argv, extra=extra))
