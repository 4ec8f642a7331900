"""The rocprofv3 summarizer (sharded_shard_amd.profiling) on synthetic
rocprofv3 output (CPU only).

Fake kernel-stats and counter CSVs with known values stand in for a profiled
run; the test checks the arithmetic the summaries rest on: request bytes
(32/64/128-byte read requests, 64-byte and 32-byte write requests), the
FETCH_SIZE / WRITE_SIZE scales fitted on a copy of known size, GB/s from
algorithmic bytes over the trace's average duration, and the traffic ratio.
"""
import csv
import json
import os

import pytest

capi = pytest.importorskip("sharded_shard_amd.capi")
from sharded_shard_amd import profiling as P  # noqa: E402

GiB2 = 2 * (1 << 30)


def _stats(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"])
        for name, calls, avg_ns in rows:
            w.writerow([name, calls, calls * avg_ns, avg_ns, avg_ns * 0.9, avg_ns * 1.1])


def _counters(path, rows):
    """rows: (kernel, counter, value) per dispatch."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for i, (k, c, v) in enumerate(rows):
            w.writerow([i, k, c, v, 0, 1000])


def _make(prof, step_bytes_factor=1.0):
    # calibration: a 2 GiB copy, FETCH_SIZE reads half its bytes (scale 2)
    big = "__amd_rocclr_copyBuffer"
    _counters(f"{prof}/cal_FETCH/x/cal_counter_collection.csv",
              [(big, "FETCH_SIZE", GiB2 / 2 / 1024), ("small", "FETCH_SIZE", 1)])
    _counters(f"{prof}/cal_WRITE/x/cal_counter_collection.csv", [(big, "WRITE_SIZE", GiB2 / 1024)])
    _counters(f"{prof}/cal_RD/x/cal_counter_collection.csv",
              [(big, "TCC_EA0_RDREQ_128B_sum", GiB2 / 128), (big, "TCC_EA0_RDREQ_sum", GiB2 / 128)])
    _counters(f"{prof}/cal_WR/x/cal_counter_collection.csv",
              [(big, "TCC_EA0_WRREQ_64B_sum", GiB2 / 64), (big, "TCC_EA0_WRREQ_sum", GiB2 / 64)])
    for tag, (ci, _, _) in P.WORKLOADS.items():
        _stats(f"{prof}/{tag}_trace/x/{tag}_kernel_stats.csv", [("unpack_kernel", 10, 100_000.0)])
        alg = P.alg_bytes_per_launch(ci, "unpack_kernel")
        rd, wr = alg / 2 * step_bytes_factor, alg / 2
        for run, rows in (("FETCH", [("unpack_kernel", "FETCH_SIZE", rd / 2 / 1024)]),
                          ("WRITE", [("unpack_kernel", "WRITE_SIZE", wr / 1024)]),
                          ("RD", [("unpack_kernel", "TCC_EA0_RDREQ_64B_sum", rd / 64),
                                  ("unpack_kernel", "TCC_EA0_RDREQ_sum", rd / 64)]),
                          ("WR", [("unpack_kernel", "TCC_EA0_WRREQ_sum", wr / 32)])):
            _counters(f"{prof}/{tag}_{run}/x/{tag}_counter_collection.csv", rows)


def test_request_bytes_by_size():
    rd, wr = P.request_bytes({"TCC_EA0_RDREQ_32B_sum": 1, "TCC_EA0_RDREQ_64B_sum": 2,
                              "TCC_EA0_RDREQ_128B_sum": 3},
                             {"TCC_EA0_WRREQ_sum": 10, "TCC_EA0_WRREQ_64B_sum": 4})
    assert rd == 32 + 128 + 384
    assert wr == 4 * 64 + 6 * 32


def test_summaries_from_synthetic_profiles(tmp_path):
    prof, out = str(tmp_path / "prof"), str(tmp_path / "out")
    _make(prof, step_bytes_factor=1.5)          # reads 1.5x the algorithmic half
    files = P.summarize(prof, out, "f" * 64)
    assert os.path.join(out, "pmc_traffic.json") in files
    cal = P.calibration(prof)
    assert cal["fetch_scale"] == pytest.approx(2.0)
    assert cal["write_scale"] == pytest.approx(1.0)
    assert cal["request_read_ratio"] == pytest.approx(1.0)
    assert cal["request_write_ratio"] == pytest.approx(1.0)
    traffic = json.load(open(os.path.join(out, "pmc_traffic.json")))
    assert traffic["kernels_source_sha256"] == "f" * 64
    for tag, (ci, _, stem) in P.WORKLOADS.items():
        alg = P.alg_bytes_per_launch(ci, "unpack_kernel")
        wl = next(w for w in traffic["workloads"].values() if w["config"] == ci)
        k = wl["kernels"]["unpack_kernel"]
        assert k["algorithmic_bytes_per_launch"] == pytest.approx(alg)
        # reads 1.5 * alg/2, writes alg/2: 1.25 x the algorithmic bytes, both ways
        assert k["traffic_bytes_per_launch"] == pytest.approx(1.25 * alg)
        assert k["traffic_fetch_write_bytes_per_launch"] == pytest.approx(1.25 * alg)
        assert k["GBps"] == pytest.approx(alg / 100e-6 / 1e9)
        md = open(os.path.join(out, f"kernels_{stem}.md")).read()
        assert "| unpack_kernel |" in md and "1.2500" in md
