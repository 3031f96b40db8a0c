"""Builds the gfx950 HIP library lib/libchunkattn.so in-tree.

Run as ``python -m chunked_spatio_temporal_amd._build``; ``__graft_entry__.build()``
calls build().  Every build recompiles from source, in three steps:

1. the device code alone (gfx950 code object in an offload bundle), with the
   compiler kept from forming packed fp32 VALU instructions
   (``-target-feature -packed-fp32-ops``, a device-only feature);
2. the host code alone, with that device binary embedded and registered at
   load time (``-fcuda-include-gpubinary``, as the HIP driver does itself);
3. the shared library from the host object and the HIP runtime.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libchunkattn.so")
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


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False, extra=()) -> str:
    """Compiles the library; `extra` flags go to both the device and host steps."""
    os.makedirs(LIBDIR, exist_ok=True)
    fatbin = LIB + ".hipfb.tmp"
    obj = LIB + ".o.tmp"
    tmp = LIB + ".tmp"
    try:
        _run([CLANG, *COMMON, *DEVICE_ONLY, *extra, SOURCE, "-o", fatbin], verbose)
        _run([CLANG, *COMMON, *HOST_ONLY, *extra, "-Xclang", "-fcuda-include-gpubinary",
              "-Xclang", fatbin, "-c", SOURCE, "-o", obj], verbose)
        _run([CLANG, "-shared", obj, "-o", tmp, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
              f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"], verbose)
        os.replace(tmp, LIB)
    finally:
        for p in (fatbin, obj, tmp):
            if os.path.exists(p):
                os.remove(p)
    return LIB


if __name__ == "__main__":
    extra = [a for a in sys.argv[1:] if a != "-v"]
    print(build(verbose="-v" in sys.argv, extra=extra))
