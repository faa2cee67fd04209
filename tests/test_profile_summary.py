"""Host logic of the rocprofv3 summary tool: per-grid aggregation and counter calibration."""
import csv
import os

from value_only_kv_amd import profile_summary as ps

TRACE_COLS = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y",
              "Grid_Size_Z", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z"]
PMC_COLS = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]


def _write(path, cols, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        w.writerows(rows)


def test_stats_separates_grids(tmp_path):
    p = tmp_path / "trace.csv"
    _write(p, TRACE_COLS, [
        ["void (anonymous namespace)::k_decode_mfma<4, 4>(gva::DecodeArgs)", 0, 1000, 512, 8, 1, 512, 1, 1],
        ["void (anonymous namespace)::k_decode_mfma<4, 4>(gva::DecodeArgs)", 0, 3000, 512, 8, 1, 512, 1, 1],
        ["void (anonymous namespace)::k_decode_mfma<4, 4>(gva::DecodeArgs)", 0, 50000, 512, 64, 1, 512, 1, 1],
    ])
    text = ps.stats(str(p), "cmd")
    assert "| `k_decode_mfma<4, 4>` | 512x8x1 | 512 | 2 | 2.00 | 2.00 | 1.00 | 3.00 |" in text
    assert "| `k_decode_mfma<4, 4>` | 512x64x1 | 512 | 1 | 50.00 | 50.00 |" in text


def test_stats_median_of_odd_and_even_counts(tmp_path):
    p = tmp_path / "trace.csv"
    name = "void (anonymous namespace)::k_combine(gva::DecodeArgs)"
    _write(p, TRACE_COLS, [[name, 0, d, 64, 1, 1, 64, 1, 1] for d in (1000, 9000, 2000)] +
                          [[name, 0, d, 128, 1, 1, 64, 1, 1] for d in (4000, 1000, 3000, 2000)])
    text = ps.stats(str(p), "cmd")
    assert "| `k_combine` | 64x1x1 | 64 | 3 | 4.00 | 2.00 | 1.00 | 9.00 |" in text
    assert "| `k_combine` | 128x1x1 | 64 | 4 | 2.50 | 2.50 | 1.00 | 4.00 |" in text


def test_traffic_calibrates_against_copy(tmp_path):
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    # the copy of 1 MiB reads 512 KiB of FETCH_SIZE (factor 2) and 1024 KiB of WRITE_SIZE
    _write(f, PMC_COLS, [["__amd_rocclr_copyBuffer", 1, "FETCH_SIZE", 512.0],
                         ["k_decode_mfma<4,4>", 4096, "FETCH_SIZE", 100.0],
                         ["k_decode_mfma<4,4>", 4096, "FETCH_SIZE", 102.0],
                         ["k_decode_mfma<4,4>", 64, "FETCH_SIZE", 9999.0]])
    _write(w, PMC_COLS, [["__amd_rocclr_copyBuffer", 1, "WRITE_SIZE", 1024.0],
                         ["k_decode_mfma<4,4>", 4096, "WRITE_SIZE", 3.0]])
    text = ps.traffic(str(f), str(w), 1 << 20, ["k_decode_mfma:4096"], 200000, "cmd")
    expect = int(round(101.0 * 1024 * 2 + 3.0 * 1024))
    assert f"traffic_bytes_per_call: {expect}" in text
    md = tmp_path / "t.md"
    md.write_text(text)
    assert ps.read_traffic(str(md), 200000) == expect
    assert ps.read_traffic(str(md), 200001) is None          # another workload
    md.write_text(text.replace(ps.sources_sha256(), "0" * 64))
    assert ps.read_traffic(str(md), 200000) is None          # kernels changed since the counters


def test_committed_traffic_profile_is_well_formed():
    path = os.path.join(os.path.dirname(__file__), "..", "profiles",
                        "gva_decode_ragged_batch_hbm_traffic.md")
    kv = {}
    for line in open(path, encoding="utf-8"):
        k, sep, v = line.partition(":")
        if sep and k in ("traffic_bytes_per_call", "algorithmic_bytes_per_call"):
            kv[k] = int(v)
    assert set(kv) == {"traffic_bytes_per_call", "algorithmic_bytes_per_call"}
    assert 1.0 <= kv["traffic_bytes_per_call"] / kv["algorithmic_bytes_per_call"] < 1.5


def test_counters_clock_and_matrix_core_busy(tmp_path):
    """Per-dispatch means, the clock from the 8 XCDs' summed GRBM_GUI_ACTIVE and the matrix-core
    busy share of an average SIMD, for the selected kernel and grid only."""
    p = tmp_path / "pmc.csv"
    cols = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value",
            "Start_Timestamp", "End_Timestamp"]
    # two dispatches of 10 us; 8 XCDs x 20000 cycles = 2.0 GHz; matrix cores busy 1024 x 5000
    rows = []
    for d in (1, 2):
        rows += [[d, "void (anonymous namespace)::k_prefill<4>(gva::PrefillArgs)", 131072,
                  "GRBM_GUI_ACTIVE", 8 * 20000.0, 0, 10000],
                 [d, "void (anonymous namespace)::k_prefill<4>(gva::PrefillArgs)", 131072,
                  "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 5000.0 * d, 0, 10000]]
    rows += [[3, "void (anonymous namespace)::k_prefill<4>(gva::PrefillArgs)", 64,
              "GRBM_GUI_ACTIVE", 1.0, 0, 10]]
    _write(p, cols, rows)
    text = ps.counters(str(p), ["k_prefill<4>:131072"], "cmd")
    line = [l for l in text.splitlines() if l.startswith("| `k_prefill<4>`")]
    assert len(line) == 1
    cells = [c.strip() for c in line[0].strip("|").split("|")]
    assert cells[1:4] == ["131072", "2", "10.00"]
    assert cells[-2:] == ["2.00", "0.375"]                  # mean busy 7500 of 20000 cycles
