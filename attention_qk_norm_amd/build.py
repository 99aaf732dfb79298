"""Build libqknorm.so (the QK-Norm library) and libqkceil.so (the
measurement kernels the benchmark times beside it) in-tree for gfx950 with
hipcc.

The shared objects land next to this file, where the Python binding and the
benchmark load them.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqknorm.so")
SOURCES = [os.path.join(CSRC, f) for f in ("qknorm_kernels_f32.hip", "qknorm_kernels_bf16.hip",
                                            "qknorm_kernels_fp8.hip", "qknorm_launch.cpp", "qknorm_api.cpp")]
CEIL_LIB = os.path.join(PKG, "libqkceil.so")
CEIL_SOURCES = [os.path.join(CSRC, "qkceil.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wextra",
    # keep the compiler from forming packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def build(out=LIB, extra=(), verbose=False, sources=None):
    """Compile every HIP source (always, in parallel: one object per source)
    and link them into `out`."""
    sources = SOURCES if sources is None else sources
    tag = "%s.tmp%d" % (out, os.getpid())
    objs = [tag + ".%d.o" % i for i in range(len(sources))]
    procs = []
    try:
        for src, obj in zip(sources, objs):
            cmd = [HIPCC, *FLAGS, *extra, "-c", "-x", "hip", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd)))
        failed = [src for src, p in procs if p.wait() != 0]
        if failed:
            raise RuntimeError("hipcc failed for " + ", ".join(failed))
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tag]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tag, out)
    finally:
        for _, p in procs:
            if p.poll() is None:
                p.kill()
                p.wait()
        for f in objs + [tag]:
            if os.path.exists(f):
                os.remove(f)
    return out


def build_ceiling(verbose=False):
    """The measurement kernels (include/qkceil.h) as libqkceil.so."""
    return build(out=CEIL_LIB, verbose=verbose, sources=CEIL_SOURCES)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_ceiling(verbose="-v" in sys.argv))
