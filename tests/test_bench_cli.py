"""bench.py's contract without a GPU: a request for several GPUs stops with a
message before anything touches a device, and the rocprofv3 summaries under
profiles/ that the benchmark reads are consistent with the workloads they
name (algorithmic bytes, the traffic ratio, the commands that made them)."""
import glob
import json
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
from attention_qk_norm_amd import workloads  # noqa: E402

BENCH = os.path.join(ROOT, "bench.py")


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_several_gpus_exit_with_a_message(argv, env):
    out = subprocess.run([sys.executable, BENCH, *argv], capture_output=True, text=True, timeout=120,
                         env={**os.environ, **env})
    assert out.returncode == 2, (out.returncode, out.stderr[-500:])
    assert "one GPU" in out.stderr
    assert out.stdout == ""


def traffic_files():
    return sorted(glob.glob(os.path.join(ROOT, "profiles", "qknorm_fwd_*_traffic.json")))


def test_profiles_present():
    names = {os.path.basename(p).split("_")[2] for p in traffic_files()}
    assert "c5" in names, names  # the default workload's traffic is what the benchmark reports


@pytest.mark.parametrize("path", traffic_files(), ids=lambda p: os.path.basename(p))
def test_traffic_summary_consistent(path):
    with open(path) as f:
        t = json.load(f)
    w = workloads.WORKLOADS[t["workload"]]
    assert t["algorithmic_bytes_per_launch"] == w.algorithmic_bytes()
    assert t["num_slices"] in w.slices
    total = t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]
    assert abs(t["bytes_per_launch"] - total) <= 1e-6 * total
    assert abs(t["traffic_over_algorithmic"] - total / w.algorithmic_bytes()) < 1e-9
    # measured traffic can exceed the algorithmic bytes (weights fetched once
    # per L2) but never fall short of them by more than counter noise
    assert 0.99 < t["traffic_over_algorithmic"] < 1.25
    for leg, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        assert t[leg]["counter"] == counter
        assert "rocprofv3 --pmc %s" % counter in t[leg]["command"]
        assert "bench.py" in t[leg]["command"] and "_work" not in t[leg]["command"]
    trace = path.replace("_traffic.json", "_kernel_trace.txt")
    assert os.path.exists(trace)
    with open(trace) as f:
        head = f.read(4000)
    assert "rocprofv3 --kernel-trace --stats" in head and "bench.py" in head
