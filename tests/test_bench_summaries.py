"""Host logic of bench.py's rocprofv3 summaries on small hand-made CSV files:
per-dispatch counter sums, per (kernel, grid) means, the MFMA-busy and clock
normalisation, and the traffic scaling by a copy of known size."""
import csv
import json
import os

import pytest

import bench

FIELDS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
          "End_Timestamp"]


def _write(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


K = "void slm::(anonymous namespace)::prefill_persistent_kernel<128, 2, false>(slm::PrefillParams)"
C = "__amd_rocclr_copyBuffer"


def test_sq_normalisation(tmp_path):
    d = str(tmp_path / "sq")
    # one dispatch of 1000 ns: 8 XCDs x 2000 cycles -> 2.0 GHz; 100 MFMAs of 32 busy cycles each over
    # 1024 SIMDs x 2000 cycles -> 3200 / 2,048,000
    _write(d, [(1, 131072, K, "GRBM_GUI_ACTIVE", 16000, 0, 1000),
               (1, 131072, K, "SQ_INSTS_MFMA", 60, 0, 1000),       # two instances of one counter add up
               (1, 131072, K, "SQ_INSTS_MFMA", 40, 0, 1000),
               (1, 131072, K, "SQ_VALU_MFMA_BUSY_CYCLES", 3200, 0, 1000),
               (1, 131072, K, "SQ_WAVES", 10, 0, 1000),
               (1, 131072, K, "SQ_INSTS_VALU", 500, 0, 1000)])
    text = bench.summarize_sq([d])
    row = json.loads(text.splitlines()[1])
    assert row["clock_GHz"] == 2.0
    assert row["MFMA_busy_cycles_per_inst"] == 32.0
    assert row["MFMA_busy_frac"] == pytest.approx(3200 / (2000 * 1024), abs=1e-4)
    assert row["VALU_per_MFMA"] == 5.0 and row["VALU_per_wave"] == 50.0


def test_traffic_scaling(tmp_path, monkeypatch):
    cf, cw, f, w = (str(tmp_path / x) for x in ("cf", "cw", "f", "w"))
    copy_kib = (1 << 30) / 1024
    _write(cf, [(1, 1, C, "FETCH_SIZE", copy_kib / 2, 0, 10)])      # FETCH_SIZE reads half the copied bytes
    _write(cw, [(1, 1, C, "WRITE_SIZE", copy_kib, 0, 10)])
    _write(f, [(5, 131072, K, "FETCH_SIZE", 1000.0, 0, 10), (6, 131072, K, "FETCH_SIZE", 3000.0, 0, 10)])
    _write(w, [(5, 131072, K, "WRITE_SIZE", 500.0, 0, 10), (6, 131072, K, "WRITE_SIZE", 500.0, 0, 10)])
    rec = str(tmp_path / "rec.json")
    text = bench.summarize_traffic(f, w, cf, cw, record=rec)
    assert "FETCH_SIZE scale 2.0000, WRITE_SIZE scale 1.0000" in text
    r = json.load(open(rec))
    assert r["per_dispatch_kib"]["persistent_fetch"] == 2000.0 and r["per_dispatch_kib"]["dispatches"] == 2
    assert r["hbm_bytes_per_launch"] == int(2000.0 * 2 * 1024 + 500.0 * 1024)
    assert r["kernel_source_sha"] == bench.src_sha(*bench.PREFILL_SOURCES)
