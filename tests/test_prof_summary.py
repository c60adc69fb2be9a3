"""Host logic of the measurement summaries (no GPU): the rocprofv3 CSV
summaries behind profiles/, and the bench's reading of the committed traffic
figure."""
import csv
import hashlib
import os
import sys
from types import SimpleNamespace

import pytest

import prof_summary as ps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECODE = "void f4kv::(anonymous namespace)::decode_kernel<4, false>(f4kv::DecodeArgs, f4kv::QPrep<4> const*)"
COPY = "__amd_rocclr_copyBuffer"


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_scales_each_counter_by_the_copy(tmp_path):
    n = 1 << 30
    kib = n / 1024
    # the copy reads half its bytes on FETCH_SIZE and all on WRITE_SIZE; small
    # copies of the harness must not be taken for the calibration copy
    _write_counters(tmp_path / "f.csv", "FETCH_SIZE",
                    [(COPY, kib / 2), (COPY, kib / 2), (COPY, 3.0), (DECODE, 1000.0), (DECODE, 1002.0),
                     ("other_kernel", 7.0)])
    _write_counters(tmp_path / "w.csv", "WRITE_SIZE",
                    [(COPY, kib), (COPY, kib), (COPY, kib), (DECODE, 10.0), (DECODE, 14.0)])
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel source")
    a = SimpleNamespace(fetch=str(tmp_path / "f.csv"), write=str(tmp_path / "w.csv"), copy_bytes=n,
                        kernel="decode_kernel<4, false>", source=str(src), cmd_fetch="F", cmd_write="W")
    out = ps.traffic(a)
    fetch = 1001.0 * 2.0 * 1024
    write = 12.0 * 1.0 * 1024
    assert f"- fetch bytes per launch: {fetch:.0f}" in out
    assert f"- write bytes per launch: {write:.0f}" in out
    assert f"- traffic bytes per launch: {fetch + write:.0f}" in out
    assert hashlib.sha256(b"kernel source").hexdigest() in out


def test_traffic_refuses_a_missing_kernel_or_copy(tmp_path):
    _write_counters(tmp_path / "f.csv", "FETCH_SIZE", [(DECODE, 1.0)])
    _write_counters(tmp_path / "w.csv", "WRITE_SIZE", [(DECODE, 1.0)])
    src = tmp_path / "k.hip"
    src.write_bytes(b"x")
    a = SimpleNamespace(fetch=str(tmp_path / "f.csv"), write=str(tmp_path / "w.csv"), copy_bytes=1 << 20,
                        kernel="decode_kernel<4, false>", source=str(src), cmd_fetch="F", cmd_write="W")
    with pytest.raises(SystemExit):
        ps.traffic(a)


def test_stats_table_lists_the_library_kernels_first_and_averages_a_window(tmp_path):
    stats = tmp_path / "run_kernel_stats.csv"
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writeheader()
        w.writerow({"Name": "at::native::big_kernel()", "Calls": 3, "AverageNs": 9e6, "MinNs": 8e6, "MaxNs": 1e7,
                    "Percentage": 60.0})
        w.writerow({"Name": DECODE, "Calls": 4, "AverageNs": 250000, "MinNs": 200000, "MaxNs": 300000,
                    "Percentage": 40.0})
    trace = tmp_path / "run_kernel_trace.csv"
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        # start order differs from file order; dispatches 2 and 3 (1-based) take 210 and 230 us
        for start, dur in [(400, 300000), (0, 200000), (100, 210000), (200, 230000)]:
            w.writerow({"Kernel_Name": DECODE, "Start_Timestamp": start, "End_Timestamp": start + dur})
    out = ps.stats_table(str(stats), "cmd", "decode_kernel<4, false>:1:2")
    body = out.split("|---|")[1]
    assert body.index("decode_kernel<4, false>") < body.index("at::native::big_kernel")
    assert "| 4 | 250.0 | 200.0 | 300.0 | 40.00% |" in out
    assert "dispatches 2 .. 3 of 4 in start order (the timed launches): average 220.0 us, min 210.0, max 230.0" in out
    with pytest.raises(SystemExit):
        ps.stats_table(str(stats), "cmd", "decode_kernel<4, false>:3:5")


def test_committed_traffic_figure_belongs_to_the_current_decode_source():
    """The bench reports the committed HBM traffic only while decode.hip is the
    source the counters were taken from; the committed summary must match it."""
    sys.path.insert(0, ROOT)
    import bench
    t = bench.measured_traffic()
    assert t is not None, "profiles/decode_kernel_traffic.md was taken from another decode.hip"
    # the algorithmic bytes of one launch (906,092,928 read from the cache), plus
    # the partial states written (~4.2 MB) and the query operands read once per
    # workgroup (~2 MB): within 1.5%, i.e. no wasted re-reads of the cache
    assert 0.99 < t / 906_092_928 < 1.015


def test_launch_shapes_split_one_kernel_by_grid(tmp_path):
    trace = tmp_path / "t_kernel_trace.csv"
    cols = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"] + [f"{k}_Size_{a}" for k in ("Workgroup", "Grid")
                                                                  for a in "XYZ"]
    pre = "void f4kv::(anonymous namespace)::prefill_kernel<false>(f4kv::PrefillArgs, int const*)"
    with open(trace, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        # grid sizes in work-items along x (256 per workgroup), workgroups along y and z
        for start, dur, gx, gz in [(0, 9000, 64 * 256, 2), (10, 1000, 3 * 256, 42), (20, 3000, 3 * 256, 42),
                                   (30, 11000, 64 * 256, 2)]:
            w.writerow({"Kernel_Name": pre, "Start_Timestamp": start, "End_Timestamp": start + dur,
                        "Workgroup_Size_X": 256, "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1,
                        "Grid_Size_X": gx, "Grid_Size_Y": 4, "Grid_Size_Z": gz})
        w.writerow({"Kernel_Name": DECODE, "Start_Timestamp": 0, "End_Timestamp": 5, "Workgroup_Size_X": 256,
                    "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1, "Grid_Size_X": 256, "Grid_Size_Y": 4,
                    "Grid_Size_Z": 1})
    out = ps.launch_shapes(str(trace), ["prefill_kernel<false>"])
    assert "| `prefill_kernel<false>` | 64 x 4 x 2 | 2 | 10.0 | 9.0 | 11.0 |" in out
    assert "| `prefill_kernel<false>` | 3 x 4 x 42 | 2 | 2.0 | 1.0 | 3.0 |" in out
    assert "decode_kernel" not in out.split("from the kernel trace:")[1]


def test_short_names_drop_namespaces_and_arguments():
    assert ps._short(DECODE) == "decode_kernel<4, false>"
    # a kernel in an anonymous namespace outside f4kv (the ceiling kernels beside bench.py)
    assert ps._short("void (anonymous namespace)::stream_read_kernel<16>(uint4 const*, long, unsigned int*)") == \
        "stream_read_kernel<16>"
