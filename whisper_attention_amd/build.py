"""Build libwa.so (the C-ABI HIP library) and libwa_diag.so (the
measurement probes of include/wa_diag.h) in-tree for gfx950.

Run as ``python whisper_attention_amd/build.py`` (by path: importing the package
would load the library before it is rebuilt); ``__graft_entry__.build()``
calls :func:`build`.  Every call compiles from source.
"""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libwa.so")
DIAG_LIB = os.path.join(PKG, "libwa_diag.so")

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # IEEE fp32 division for the quantize step's x / scale (no fast-math)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _link(srcs, lib, verbose, extra):
    tmp = lib + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the device-only target feature; drop that note
    out = "\n".join(ln for ln in res.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if out.strip() and verbose:
        print(out)
    os.replace(tmp, lib)
    return lib


def build(verbose=False, extra=()):
    _link(sorted(glob.glob(os.path.join(PKG, "csrc", "diag", "*.hip"))), DIAG_LIB, verbose, extra)
    return _link(sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip"))), LIB, verbose, extra)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
