"""The C ABI from a C++ caller (tests/c_abi_check.cpp): device buffers from
hipMalloc, every entry point of include/qknorm.h (fused forward with default
and forced options, headwise, inverse RMS, the split path for one tensor and
for both at once) against the fp64 oracle, and the documented error codes,
status strings and width limits, with no Python in between."""
import os
import subprocess

import pytest

import c_abi_build

pytestmark = pytest.mark.gpu


def test_c_caller():
    if not os.path.exists(c_abi_build.EXE):  # normally built by __graft_entry__.build()
        c_abi_build.build()
    print("[case] c_abi_check", flush=True)
    out = subprocess.run([c_abi_build.EXE], capture_output=True, text=True, timeout=120)
    print(out.stdout, flush=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "c_abi_check: ok" in out.stdout
