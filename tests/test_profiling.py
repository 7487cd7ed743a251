"""Host tests of the rocprofv3 CSV summaries (no GPU): the traffic figure is the profiled
kernel's FETCH_SIZE / WRITE_SIZE scaled by what the counters read for a calibration copy."""
import csv
import json
from types import SimpleNamespace

from memory_bound_decode_add_amd import profiling

FIELDS = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for name, grid, value in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_calibrates_on_the_largest_copy(tmp_path):
    gemv = "void fdec::w4_gemv_col_kernel<1, 2, 5, 1>(ColArgs)"
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    big, small = 512 << 20, 12 << 20
    # FETCH_SIZE reads half the bytes, WRITE_SIZE all of them; the small copy (a warm-up
    # between timed rounds) has its own, different counter values and must be ignored
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(gemv, 262144, 6000.0), (gemv, 262144, 6200.0),
                                           (copy, 33554432, big / 2048), (copy, 381440, 1000.0)] +
         [(copy, 381440, 2000.0)] * 5)
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(gemv, 262144, 5.0), (gemv, 262144, 5.0),
                                           (copy, 33554432, big / 1024), (copy, 381440, small / 1024)])
    out = tmp_path / "t.json"
    a = SimpleNamespace(fetch=str(tmp_path / "f.csv"), write=str(tmp_path / "w.csv"), kernel="w4_gemv_col_kernel",
                        copy="neg_kernel", copy_read_bytes=big, copy_write_bytes=big, bytes_per_launch=12_000_000,
                        command_fetch="cf", command_write="cw", out=str(out))
    profiling.traffic(a)
    doc = json.loads(out.read_text())
    assert doc["fetch_scale"] == 2.0 and doc["write_scale"] == 1.0
    assert doc["hbm_bytes_per_launch"] == (6100.0 * 2 + 5.0) * 1024
    assert doc["kernel"] == gemv


def test_traffic_rejects_an_ambiguous_kernel(tmp_path):
    k = "void fdec::w4_gemv_col_kernel<1, 2, 5, 1>(ColArgs)"
    copy = "neg_kernel_cuda"
    for name, counter in (("f.csv", "FETCH_SIZE"), ("w.csv", "WRITE_SIZE")):
        _csv(tmp_path / name, counter, [(k, 262144, 1.0), (k, 131072, 1.0), (copy, 1024, 1.0)])
    a = SimpleNamespace(fetch=str(tmp_path / "f.csv"), write=str(tmp_path / "w.csv"), kernel="w4_gemv_col_kernel",
                        copy="neg_kernel", copy_read_bytes=1024, copy_write_bytes=1024, bytes_per_launch=1,
                        command_fetch="cf", command_write="cw", out=str(tmp_path / "t.json"))
    try:
        profiling.traffic(a)
    except SystemExit as e:
        assert "2 kernel shapes" in str(e)
    else:
        raise AssertionError("two launch shapes of the profiled kernel must be rejected")
