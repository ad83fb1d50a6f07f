"""bench_profiles.py on small synthetic rocprofv3 CSVs (no GPU): the copy
calibration scales FETCH_SIZE and WRITE_SIZE to bytes, the per-launch figures
are means over the matching dispatches, and the busy fractions follow the
counter definitions."""
import csv
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench_profiles  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Start_Timestamp",
          "End_Timestamp", "Counter_Name", "Counter_Value"]


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _row(did, name, grid, us, counter, value):
    return {"Dispatch_Id": did, "Kernel_Name": name, "Grid_Size": grid, "Workgroup_Size": 256,
            "Start_Timestamp": 1000, "End_Timestamp": 1000 + int(us * 1000),
            "Counter_Name": counter, "Counter_Value": value}


def test_calibrated_traffic_and_busy_fractions(tmp_path):
    copy, kern = "__amd_rocclr_copyBuffer", "void (anonymous namespace)::my_kernel(int)"
    # the copy reads 256 MiB: FETCH_SIZE counts half of it (scale 2), WRITE_SIZE all
    _write(str(tmp_path / "pmc_fetch" / "run_counter_collection.csv"),
           [_row(1, copy, 131072, 40, "FETCH_SIZE", 131072.0),
            _row(2, kern, 4096, 10, "FETCH_SIZE", 1000.0),
            _row(3, kern, 4096, 10, "FETCH_SIZE", 3000.0)])
    _write(str(tmp_path / "pmc_write" / "run_counter_collection.csv"),
           [_row(1, copy, 131072, 40, "WRITE_SIZE", 262144.0),
            _row(2, kern, 4096, 10, "WRITE_SIZE", 500.0),
            _row(3, kern, 4096, 10, "WRITE_SIZE", 700.0)])
    sq = []
    for did in (2, 3):
        # 100 us at 2.0 GHz on 8 XCDs: GRBM_GUI_ACTIVE = 8 * 200000 cycles
        for name, v in (("GRBM_GUI_ACTIVE", 8 * 200000.0),
                        ("SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 200000 * 1024),
                        ("SQ_ACTIVE_INST_VALU", 0.5 * 200000 * 1024 / 4),
                        ("SQ_INSTS_VALU", 10.0), ("SQ_INSTS_VALU_TRANS_F32", 2.0),
                        ("SQ_INSTS_MFMA", 3.0), ("SQ_INSTS_LDS", 4.0)):
            sq.append(_row(did, kern, 4096, 100, name, v))
    _write(str(tmp_path / "pmc_sq" / "run_counter_collection.csv"), sq)
    c = bench_profiles.Counters(str(tmp_path))
    assert abs(c.sf - 2.0) < 1e-12 and abs(c.sw - 1.0) < 1e-12
    f, w, fb, wb = c.traffic("my_kernel", 4096)
    assert f == [1000.0, 3000.0] and w == [500.0, 700.0]
    assert fb == 2000.0 * 1024 * 2.0 and wb == 600.0 * 1024
    _, m = c.sq_block(bench_profiles.ordered(c.smeta, "my_kernel", 4096), "my_kernel")
    assert abs(m["clock_ghz"] - 2.0) < 1e-9
    assert abs(m["mfma_busy"] - 0.25) < 1e-12 and abs(m["valu_active"] - 0.5) < 1e-12


def test_source_fingerprint_matches_bench():
    import bench
    assert bench_profiles.sha(bench_profiles.FUSED) == bench._sources_hash(bench.FUSED_SOURCES)
    assert bench_profiles.SSM == bench.SSM_SOURCES and bench_profiles.STEP == bench.STEP_SOURCES
    assert bench_profiles.ATTN == bench.ATTN_SOURCES and bench_profiles.LIN == bench.LINEAR_SOURCES
