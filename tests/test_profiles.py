"""The committed HBM-traffic records agree with bench.py.

bench.py reports a kernel's measured traffic only from a record taken on the
kernel's current sources (a digest over the files it lists). These checks
keep the records well formed: each names a kernel bench.py knows, lists
exactly that kernel's source files (all present), carries counters and copy
calibration factors that reproduce its stored traffic figure, and lies
within a few percent of its algorithmic bytes or at a whole multiple of
them (a pass that reads its rows more than once).
"""

import glob
import json
import os

import pytest

import bench

RECORDS = sorted(glob.glob(os.path.join(bench.PROFILES, "traffic_*.json")))


def test_records_exist():
    assert len(RECORDS) >= 4


@pytest.mark.parametrize("path", RECORDS, ids=[os.path.basename(p) for p in RECORDS])
def test_record_is_consistent(path):
    with open(path) as f:
        t = json.load(f)
    assert t["kernel"] in bench.STREAM_SOURCES
    assert t["source_files"] == list(bench.STREAM_SOURCES[t["kernel"]])
    for name in t["source_files"]:
        assert os.path.exists(os.path.join(bench.CSRC, name))
    assert os.path.basename(path) == os.path.basename(bench.traffic_file(t["kernel"], t["workload"]))
    scaled = (t["fetch_kib_per_dispatch"] * 1024.0 * t["copy_factor_fetch"]
              + t["write_kib_per_dispatch"] * 1024.0 * t["copy_factor_write"])
    assert abs(scaled - t["traffic_bytes_per_dispatch"]) <= 1e-6 * scaled + 1.0
    ratio = scaled / t["algorithmic_bytes_per_dispatch"]
    assert abs(ratio - round(ratio)) < 0.05 and round(ratio) >= 1
    for cmd in t["commands"]:
        assert "bench.py" in cmd and "_work" not in cmd
