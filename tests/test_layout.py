"""The launch planner and slot tables, checked on the host (no GPU): the
library's host source is compiled together with tests/layout_check.cpp,
which replaces the device launch and checks every planned layout through
the same slot_vector() function the kernels use. It also prints the plan of
each benchmark workload, pinned here: a planner change that moves one of
them fails until the pin is updated on purpose, with its measurement."""
import os
import subprocess

import pytest

from conftest import ROOT

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# team = wavefronts per row, sub_lanes = lanes that deal one slice, slots =
# 16-byte vectors per lane, body = the compiled slot count the launch runs
WORKLOAD_PLANS = [
    'plan c1 K=1: nw=4 body=1 narrow=0 rows_per_wave=1 paired=0 early=0 | q team=4 sub_lanes=64 slots=1 masked=0 | k team=4 sub_lanes=64 slots=1 masked=0',
    'plan c1 K=4: nw=4 body=1 narrow=0 rows_per_wave=1 paired=0 early=0 | q team=4 sub_lanes=64 slots=1 masked=0 | k team=4 sub_lanes=64 slots=1 masked=0',
    'plan c2 K=1: nw=4 body=2 narrow=0 rows_per_wave=1 paired=0 early=0 | q team=4 sub_lanes=256 slots=2 masked=0 | k team=4 sub_lanes=256 slots=2 masked=0',
    'plan c3 K=4: nw=4 body=3 narrow=0 rows_per_wave=1 paired=0 early=0 | q team=4 sub_lanes=64 slots=3 masked=0 | k team=4 sub_lanes=64 slots=3 masked=0',
    'plan c3 K=1: nw=4 body=3 narrow=0 rows_per_wave=1 paired=0 early=0 | q team=4 sub_lanes=256 slots=3 masked=0 | k team=4 sub_lanes=256 slots=3 masked=0',
    'plan c4 K=1: nw=4 body=10 narrow=0 rows_per_wave=1 paired=2 early=0 | q team=1 sub_lanes=64 slots=10 masked=0 | k team=1 sub_lanes=64 slots=2 masked=0',
    'plan c5 K=8: nw=4 body=4 narrow=0 rows_per_wave=1 paired=0 early=0 | q team=2 sub_lanes=64 slots=4 masked=0 | k team=2 sub_lanes=64 slots=4 masked=0',
    'plan c5 K=1: nw=4 body=4 narrow=0 rows_per_wave=1 paired=0 early=0 | q team=2 sub_lanes=128 slots=4 masked=0 | k team=2 sub_lanes=128 slots=4 masked=0',
    'plan c4f8 K=1: nw=4 body=5 narrow=0 rows_per_wave=1 paired=1 early=1 | q team=1 sub_lanes=64 slots=5 masked=0 | k team=1 sub_lanes=64 slots=1 masked=0',
    'plan c5f8 K=8: nw=4 body=4 narrow=1 rows_per_wave=1 paired=0 early=0 | q team=1 sub_lanes=8 slots=4 masked=0 | k team=1 sub_lanes=8 slots=4 masked=0',
    'plan c5f8 K=1: nw=4 body=4 narrow=0 rows_per_wave=1 paired=0 early=0 | q team=1 sub_lanes=64 slots=4 masked=0 | k team=1 sub_lanes=64 slots=4 masked=0',
]


@pytest.fixture(scope="module")
def checker_output(tmp_path_factory):
    exe = os.path.join(tmp_path_factory.mktemp("layout"), "layout_check")
    subprocess.run([HIPCC, "-O1", "-std=c++17", "-x", "hip", "--cuda-host-only",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "attention_qk_norm_amd", "csrc"),
                    os.path.join(ROOT, "tests", "layout_check.cpp"), "-o", exe],
                   check=True, stderr=subprocess.DEVNULL)
    out = subprocess.run([exe], capture_output=True, text=True)
    return out.returncode, out.stdout


def test_layouts_cover_every_vector_once(checker_output):
    rc, out = checker_output
    assert rc == 0, out[-3000:]
    assert out.strip().endswith("0 failures"), out[-3000:]


def test_workload_plans_unchanged(checker_output):
    _, out = checker_output
    got = [line for line in out.splitlines() if line.startswith("plan ")]
    assert got == WORKLOAD_PLANS
