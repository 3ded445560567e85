"""bench.py's counter summary (CPU only): two synthetic rocprofv3 counter files
with a 1 GiB calibration copy turn into per-call HBM bytes of aba_attend, and the
record is reported only while attend.hip is unchanged."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.abspath(os.path.join(os.path.dirname(__file__), ".."))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

COLS = ["Correlation_Id", "Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]
ATTEND = ("void aba::(anonymous namespace)::attend_bf16_kernel<128, false>(unsigned short const*, int, float, "
          "bool)")
ORDER = "aba::(anonymous namespace)::order_kernel(int const*, int, int, int, int*)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(COLS)
        for i, (name, grid, value) in enumerate(rows):
            w.writerow([i + 1, i + 1, grid, name, counter, value])


def test_summary_scales_by_the_calibration_copy(tmp_path):
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    # FETCH_SIZE reads half of the bytes a copy moves (scale 2), WRITE_SIZE all of them (scale 1)
    _write(fetch, "FETCH_SIZE", [(COPY, 1, 524288.0), (ORDER, 8192, 30.0), (ATTEND, 786432, 800000.0),
                                 (ATTEND, 786432, 900000.0), (COPY, 1, 4.0)])
    _write(write, "WRITE_SIZE", [(COPY, 1, 1048576.0), (ORDER, 8192, 12.0), (ATTEND, 786432, 100000.0),
                                 (ATTEND, 786432, 100000.0)])
    out = tmp_path / "profiles"
    out.mkdir()
    rec = bench.summarize_traffic(fetch, write, 128, ["cmd one", "cmd two"], out_dir=str(out))
    att = rec["kernels"]["void aba::attend_bf16_kernel<128, false>"]
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert att["read_bytes"] == pytest.approx(850000.0 * 1024 * 2)        # mean of the two launches, scaled
    assert att["write_bytes"] == pytest.approx(100000.0 * 1024)
    assert rec["bytes_per_launch"] == pytest.approx((850000.0 + 30.0) * 2048 + (100000.0 + 12.0) * 1024)
    md = (out / "hbm_traffic_single_layer.md").read_text()
    assert "cmd one" in md and "x2.0000" in md
    path = str(out / "attend_single_layer_traffic.json")
    assert bench.traffic_entry(128, path) == pytest.approx(rec["bytes_per_launch"])
    # a record taken with another attend.hip is not reported
    stale = dict(rec, attend_src_sha256_16="0" * 16)
    json.dump(stale, open(path, "w"))
    assert bench.traffic_entry(128, path) is None


def test_summary_needs_the_calibration_copy(tmp_path):
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    _write(fetch, "FETCH_SIZE", [(ORDER, 8192, 30.0), (ATTEND, 786432, 800000.0)])
    _write(write, "WRITE_SIZE", [(ORDER, 8192, 12.0), (ATTEND, 786432, 100000.0)])
    with pytest.raises(SystemExit):
        bench.summarize_traffic(fetch, write, 128, [], out_dir=str(tmp_path))
