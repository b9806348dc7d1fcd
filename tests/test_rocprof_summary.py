"""The profile summary tool and the benchmark's readers of committed
summaries, on hand-written rocprofv3-style CSV files (no GPU)."""

import csv
import json

import pytest

import bench
from paged_kv_cache_178_amd import rocprof_summary as rs


def write_counters(path, kernel, values):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for d, per in enumerate(values):
            for name, v in per.items():
                w.writerow({"Dispatch_Id": d, "Kernel_Name": kernel, "Counter_Name": name,
                            "Counter_Value": v})


def test_mfma_busy_is_busy_over_active_simd_cycles():
    # 8 XCCs of 1000 active cycles each (the per-dispatch value sums them),
    # 1024 SIMDs busy 250 cycles each: 25%.
    vals = {"SQ_VALU_MFMA_BUSY_CYCLES": [1024 * 250.0], "GRBM_GUI_ACTIVE": [8 * 1000.0]}
    assert rs.mfma_busy_frac(vals, 1024, 8) == pytest.approx(0.25)
    assert rs.mfma_busy_frac(vals, 0, 8) is None
    assert rs.mfma_busy_frac({"GRBM_GUI_ACTIVE": [1.0]}, 1024, 8) is None


def test_counters_summary_is_stamped_and_read_back(tmp_path, monkeypatch):
    a, b = tmp_path / "a.csv", tmp_path / "b.csv"
    # Medians over three dispatches: busy 1024 * 300, active 8 * 1000 -> 30%.
    write_counters(a, "paged_prefill_kernel<2, 16>",
                   [{"SQ_VALU_MFMA_BUSY_CYCLES": 1024 * x} for x in (290, 300, 310)])
    write_counters(b, "paged_prefill_kernel<2, 16>",
                   [{"GRBM_GUI_ACTIVE": 8 * x} for x in (990, 1000, 1020)])
    out = tmp_path / "counters.md"
    sha = bench.prefill_source_sha()
    rs.main(["counters", str(a), str(b), "--kernel", "paged_prefill_kernel", "--out", str(out),
             "--cmd", "cmd", "--simds", "1024", "--xccs", "8", "--sha", sha])
    text = out.read_text()
    assert "MFMA busy: 30.0%" in text
    assert bench.stored_mfma_busy(str(out)) == pytest.approx(0.30)
    # A summary taken on other sources is not used.
    out.write_text(text.replace(sha, "0" * 16))
    assert bench.stored_mfma_busy(str(out)) is None


def test_traffic_summary_scaled_by_the_copy(tmp_path):
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # Kernel: 100 KiB fetched, 10 KiB written per dispatch; the copy of
    # 1 MiB reads as 512 KiB fetched and 1024 KiB written.
    with open(fetch, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for d in range(3):
            w.writerow({"Dispatch_Id": d, "Kernel_Name": "paged_decode_kernel<...>",
                        "Counter_Name": "FETCH_SIZE", "Counter_Value": 100})
            w.writerow({"Dispatch_Id": 10 + d, "Kernel_Name": "__amd_rocclr_copyBuffer",
                        "Counter_Name": "FETCH_SIZE", "Counter_Value": 512})
    with open(write, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for d in range(3):
            w.writerow({"Dispatch_Id": d, "Kernel_Name": "paged_decode_kernel<...>",
                        "Counter_Name": "WRITE_SIZE", "Counter_Value": 10})
            w.writerow({"Dispatch_Id": 10 + d, "Kernel_Name": "__amd_rocclr_copyBuffer",
                        "Counter_Name": "WRITE_SIZE", "Counter_Value": 1024})
    out = tmp_path / "pmc.md"
    rs.main(["pmc", "--fetch", str(fetch), "--write", str(write), "--kernel",
             "paged_decode_kernel", "--copy-kernel", "copyBuffer", "--copy-bytes",
             str(1 << 20), "--kv-bytes", str(200 * 1024), "--sha", bench.kernel_source_sha(),
             "--out", str(out), "--cmd", "cmd"])
    rec = bench.stored_traffic(str(out))
    # 100 KiB x 2048 B per counted KiB + 10 KiB x 1024 B.
    assert rec["traffic_bytes_per_launch"] == 100 * 2048 + 10 * 1024
    assert json.loads(out.read_text().split("traffic-json: ")[1])["kv_bytes_per_launch"] == 204800
