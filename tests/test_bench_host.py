"""Host logic of bench.py (no GPU): turning rocprofv3 counter CSVs into bytes.

The counters are KiB per dispatch; each is scaled so that the calibration copy
of COPY_BYTES reads (and writes) COPY_BYTES. Synthetic CSVs with known values
check the scaling, the per-shape medians (launches outside the timed step, such
as the greedy verify over every row, share a shape with the step's own) and
that only the warp's fast-path kernel feeds the roofline figure.
"""
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for name, grid, kib in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter, "Counter_Value": kib})


def test_traffic_from_counters(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    coop = "void sv::(anonymous namespace)::warp_coop_kernel<true>(unsigned short const*, int)"
    filt = "void sv::(anonymous namespace)::warp_filter_kernel<true, true>(void const*, int)"
    greedy = "void sv::(anonymous namespace)::greedy_sliced_kernel<true, false>(void const*, int)"
    copy = "__amd_rocclr_copyBuffer"
    # FETCH_SIZE sees half of every read, WRITE_SIZE all of every write
    fetch = [(coop, 1000, 100.0), (coop, 1000, 110.0), (coop, 2000, 300.0), (filt, 3000, 999.0),
             (greedy, 4000, 10.0), (greedy, 4000, 10.0), (greedy, 4000, 12.0), (greedy, 4000, 500.0),
             (copy, 64, copy_kib / 2), (copy, 64, copy_kib / 2), (copy, 64, 1.0)]
    write = [(coop, 1000, 50.0), (coop, 1000, 50.0), (coop, 2000, 70.0), (filt, 3000, 5.0),
             (copy, 64, copy_kib), (copy, 64, 2.0)]
    fp, wp, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    write_csv(fp, "FETCH_SIZE", fetch)
    write_csv(wp, "WRITE_SIZE", write)
    bench.traffic_from_counters(str(fp), str(wp), "wl", str(out))
    rec = json.loads(out.read_text())
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    # warp: shape 1000 gives 105 KiB fetched (median of 100 and 110), shape 2000 300 KiB; the two shapes averaged, x2
    assert rec["fetch_bytes_per_launch"] == int((105 + 300) / 2 * 1024 * 2)
    assert rec["write_bytes_per_launch"] == int((50 + 70) / 2 * 1024)
    assert rec["bytes_per_launch"] == rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["per_grid"]["1000"] == {"fetch": int(105 * 1024 * 2), "write": 50 * 1024}
    # the filtered warp is recorded on its own, never mixed into the roofline figure
    assert rec["kernels"]["warp_filter_kernel"]["3000"] == {"fetch": int(999 * 1024 * 2), "write": 5 * 1024}
    # the step's greedy launches, not the one full read that shares their shape
    assert rec["kernels"]["greedy_sliced_kernel"]["4000"]["fetch"] == int(11.0 * 1024 * 2)
    assert rec["kernel_source_sha"] == bench.kernel_source_sha()
    assert rec["library_source_sha"] == bench.kernel_source_sha(all_sources=True)


def test_cpu_baseline_reports_all_core_and_single_thread_medians():
    import synth
    for name in ("logits-bf16-b256-k5-v128256", "probs-b64-k4-v32000"):
        batch = synth.generate(name, "cpu", B=6, V=640)
        rec = bench.cpu_baseline(batch, 0.2)
        st = rec["single_thread"]
        assert rec["kind"] == st["kind"] == "oracle" and rec["unit"] == st["unit"] == "rounds/s"
        assert st["cores"] == 1 and rec["cores"] >= 1
        assert rec["value"] > 0 and st["value"] > 0
        assert "median of" in rec["sample"] and "of 6 sequences" in st["sample"]
