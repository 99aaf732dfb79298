"""The launch planner and slot tables, checked on the host (no GPU): the
library's host source is compiled together with tests/layout_check.cpp,
which replaces the device launch and checks every planned layout through
the same slot_vector() function the kernels use."""
import os
import subprocess

from conftest import ROOT

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_layouts_cover_every_vector_once(tmp_path):
    exe = os.path.join(tmp_path, "layout_check")
    subprocess.run([HIPCC, "-O1", "-std=c++17", "-x", "hip", "--cuda-host-only",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "attention_qk_norm_amd", "csrc"),
                    os.path.join(ROOT, "tests", "layout_check.cpp"), "-o", exe],
                   check=True, stderr=subprocess.DEVNULL)
    out = subprocess.run([exe], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout[-3000:]
    assert out.stdout.strip().endswith("0 failures"), out.stdout[-3000:]
