"""The committed HBM-traffic summaries under profiles/ belong to the kernels as
they are: each file's source digest equals the digest bench.py computes from
the current kernel sources (comments and blank lines aside), so the traffic
figure bench.py reports beside a roofline was measured on this code.  Runs on
the CPU; imports bench.py only for its digest and file readers."""
import glob
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FILES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.txt")))


def _fields(path):
    vals = {}
    for line in open(path, encoding="utf-8"):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            vals[k] = v
    return vals


def test_traffic_files_exist():
    assert FILES, "no traffic summaries under profiles/"


@pytest.mark.parametrize("path", FILES, ids=[os.path.basename(p) for p in FILES])
def test_traffic_file_matches_current_kernel(path):
    name = os.path.basename(path)[: -len("_traffic.txt")]
    pass_name, workload = name.rsplit("_w", 1)
    vals = _fields(path)
    assert pass_name in bench.KERNEL_SOURCES, name
    assert vals["source_digest"] == bench.source_digest(pass_name), (
        f"{name}: kernel sources changed since the counters were taken; re-measure FETCH_SIZE/WRITE_SIZE")
    total = int(vals["hbm_bytes_per_launch"])
    # each figure is rounded to whole bytes on its own
    assert abs(total - int(vals["read_bytes_per_launch"]) - int(vals["write_bytes_per_launch"])) <= 1
    assert bench.read_traffic(pass_name, int(workload)) == total
