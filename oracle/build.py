"""Compile the fp64 CPU oracle (test infrastructure only) with gcc.

The oracle is a checker: the product library never links it. This script is
called by the repository's build entry point and, if the shared object is
missing, by the oracle loader.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qknorm_oracle.c")
LIB = os.path.join(HERE, "libqknorm_oracle.so")


def build(src=SRC, out=LIB, extra_flags=()):
    """Compile `src` into the shared object `out`; returns `out`."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra", "-Werror", *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
