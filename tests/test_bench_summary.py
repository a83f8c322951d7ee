"""The profile summariser of bench.py on synthetic rocprofv3 CSV output (CPU
only): the calibration copy is found by its size among copies that share its
grid, FETCH and WRITE readings are paired by dispatch id, and the per-workload
traffic table scales every kernel by the copy's factors."""
import csv
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

COPY = "__amd_rocclr_copyBuffer"
GAE = "void rlscan::scan_kernel<rlscan::GaeOp<3u, false>, 8, 2, false, true>(rlscan::GaeOp<3u, false>, rlscan::Geo, unsigned char*)"
VTR = "void rlscan::scan_kernel<rlscan::VtraceOp<16u, false>, 8, 2, false, true>(rlscan::VtraceOp<16u, false>, rlscan::Geo, unsigned char*)"


def _write_counters(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for did, grid, name, val in rows:
            w.writerow([did, grid, name, counter, val])


def _write_trace(d):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_kernel_stats.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"])
        w.writerow([GAE, 10, 207000, 20700, 18000, 25000])
    with open(os.path.join(d, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size", "Start_Timestamp", "End_Timestamp"])
        w.writerow([GAE, 524288, 0, 20700])


def test_summary_picks_the_calibration_copy_by_size(tmp_path):
    kib = bench.COPY_BYTES / 1024
    big = 134217728 / 1024  # a larger copy with the same grid (an input clone)
    clone = 16777216 / 1024
    # dispatch ids: 1-3 clones, 4-5 calibration copies, 6 the larger copy, 7-8 kernels
    write = [(1, 131072, COPY, clone), (2, 131072, COPY, clone), (3, 131072, COPY, clone),
             (4, 131072, COPY, kib), (5, 131072, COPY, kib), (6, 131072, COPY, big),
             (7, 524288, GAE, 32768.0), (8, 524288, VTR, 32768.0)]
    # FETCH_SIZE reads half of the reads on this part: the copy reads kib/2
    fetch = [(1, 131072, COPY, clone / 2), (2, 131072, COPY, clone / 2), (3, 131072, COPY, clone / 2),
             (4, 131072, COPY, kib / 2), (5, 131072, COPY, kib / 2), (6, 131072, COPY, big / 2),
             (7, 524288, GAE, 84 * 1024 * 1024 / 1024 / 2), (8, 524288, VTR, 67108864 / 1024 / 2)]
    _write_counters(str(tmp_path / "fetch"), "FETCH_SIZE", fetch)
    _write_counters(str(tmp_path / "write"), "WRITE_SIZE", write)
    _write_trace(str(tmp_path / "trace"))
    out = tmp_path / "out"
    bench.summarize_profile(str(tmp_path / "trace"), str(tmp_path / "fetch"), str(tmp_path / "write"),
                            str(out), "test")
    text = (out / "scan_kernels_bench_default_kernel_trace.md").read_text()
    assert "scale factors 2.0000 (fetch) and 1.0000 (write)" in text
    # GAE: 88,080,384 B read (84 MiB) + 33,554,432 written
    traffic = (out / os.path.basename(bench.TRAFFIC_FILE)).read_text()
    assert "hbm_bytes_per_launch: 121634816" in traffic
    assert f"source_hash: {bench.source_hash()}" in traffic
    # the per-workload table holds both kernels, each scaled by the same factors
    assert "| gae_truncations_4096x1024 |" in text
    assert "| vtrace_1024x4096 | `scan_kernel<VtraceOp<16u, false>, 8, 2, false, true>` | 67108864 | 33554432 |" in text


def test_summary_without_a_calibration_copy_writes_no_traffic(tmp_path):
    write = [(1, 131072, COPY, 16384.0), (2, 524288, GAE, 32768.0)]
    fetch = [(1, 131072, COPY, 8192.0), (2, 524288, GAE, 41000.0)]
    _write_counters(str(tmp_path / "fetch"), "FETCH_SIZE", fetch)
    _write_counters(str(tmp_path / "write"), "WRITE_SIZE", write)
    _write_trace(str(tmp_path / "trace"))
    out = tmp_path / "out"
    bench.summarize_profile(str(tmp_path / "trace"), str(tmp_path / "fetch"), str(tmp_path / "write"),
                            str(out), "test")
    assert not (out / os.path.basename(bench.TRAFFIC_FILE)).exists()
    assert "HBM traffic" not in (out / "scan_kernels_bench_default_kernel_trace.md").read_text()


def test_summary_tabulates_the_sq_counter_pass(tmp_path):
    sq = tmp_path / "sq"
    os.makedirs(sq)
    with open(sq / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for did, val in ((1, 10.0), (2, 14.0), (3, 12.0)):
            for name, v in (("VALUBusy", val), ("OccupancyPercent", 45.0), ("SQ_INSTS_VALU", 2220032.0),
                            ("SQ_WAVES", 8192.0), ("MemUnitStalled", 0.5)):
                w.writerow([did, GAE, name, v])
        w.writerow([4, COPY, "VALUBusy", 1.0])  # not a library kernel: left out
    write = [(1, 131072, COPY, 16384.0), (2, 524288, GAE, 32768.0)]
    fetch = [(1, 131072, COPY, 8192.0), (2, 524288, GAE, 41000.0)]
    _write_counters(str(tmp_path / "fetch"), "FETCH_SIZE", fetch)
    _write_counters(str(tmp_path / "write"), "WRITE_SIZE", write)
    _write_trace(str(tmp_path / "trace"))
    out = tmp_path / "out"
    bench.summarize_profile(str(tmp_path / "trace"), str(tmp_path / "fetch"), str(tmp_path / "write"),
                            str(out), "test", str(sq))
    text = (out / "scan_kernels_bench_default_kernel_trace.md").read_text()
    assert "## SQ counters" in text
    # 2,220,032 VALU instructions over 8192 waves = 271 per wave; median VALU busy 12.0
    assert "| `scan_kernel<GaeOp<3u, false>, 8, 2, false, true>` | 3 | 271 | 12.0 | 45.0 | 0.50 |" in text
    assert "copyBuffer" not in text.split("## SQ counters")[1]
