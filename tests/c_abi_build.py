"""Build tests/c_abi_check.cpp, a C++ caller of libqknorm through
include/qknorm.h, linked with the library and with the fp64 oracle (test
infrastructure). __graft_entry__.build() calls this after building both."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_check.cpp")
EXE = os.path.join(HERE, "c_abi_check.bin")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(out=EXE):
    cmd = [HIPCC, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", SRC,
           "-I", os.path.join(ROOT, "include"),
           "-L", os.path.join(ROOT, "attention_qk_norm_amd"), "-lqknorm",
           "-L", os.path.join(ROOT, "oracle"), "-lqknorm_oracle",
           "-Wl,-rpath,$ORIGIN/../attention_qk_norm_amd:$ORIGIN/../oracle", "-o", out + ".tmp"]
    subprocess.run(cmd, check=True, timeout=300)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
