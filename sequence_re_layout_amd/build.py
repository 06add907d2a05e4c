"""Build ``libbasp.so`` in-tree with hipcc for gfx950 (MI355X).

    python -m sequence_re_layout_amd.build

The library is the product: the HIP kernels and the C ABI declared in
``include/basp.h``.  The Python binding loads it from this directory.
"""
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbasp.so")
SOURCES = [os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "launch.cpp"),
           os.path.join(CSRC, "relayout.hip")]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every source into libbasp.so (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-command-line-argument",
           # packed fp32 instructions stay off in all device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, "-I", CSRC] + SOURCES + ["-o", tmp]
    t0 = time.time()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built %s in %.1f s" % (LIB, time.time() - t0), flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
