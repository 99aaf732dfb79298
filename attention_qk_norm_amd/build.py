"""Build libqknorm.so in-tree for gfx950 with hipcc.

The shared object lands next to this file, where the Python binding loads it.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqknorm.so")
SOURCES = [os.path.join(CSRC, "qknorm_kernels.hip"), os.path.join(CSRC, "qknorm_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wextra",
    # keep the compiler from forming packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def build(out=LIB, extra=(), verbose=False):
    """Compile every HIP source into `out` (always recompiles)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    finally:
        if os.path.exists(tmp):
            os.remove(tmp)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
