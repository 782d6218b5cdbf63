"""CPU tests of the measurement tooling: the profiled-kernel classifier that keys the
HBM-traffic and SQ-counter summaries (and the benchmark's traffic lookup)."""
import pytest

from exact_attention_102_amd.traffic import classify


@pytest.mark.parametrize("name,expected", [
    ("void fa::fwd_kernel<128, 128, 32, 4, 3, false, false>(fa::FwdArgs)", ("fwd", "full")),
    ("void fa::fwd_kernel<128, 128, 32, 4, 3, true, false>(fa::FwdArgs)", ("fwd", "causal")),
    ("void fa::dq_kernel<128, 128, 64, 8, 2, false, false>(fa::BwdArgs)", ("dq", "full")),
    ("void fa::dkdv_kernel<128, 128, 32, 8, true, true, 2, true, false>(fa::BwdArgs)", ("dkdv_atomic", "causal")),
    ("void fa::dkdv_kernel<256, 256, 32, 4, false, false, 2, false, false>(fa::BwdArgs)", ("dkdv", "full")),
    # wide kernels: <D, DV, BQ, waves, CAUSAL, ATOMIC>
    ("void fa::dkdv_wide_kernel<128, 128, 32, 4, false, true>(fa::BwdArgs)", ("dkdv_atomic", "full")),
    ("void fa::dkdv_wide_kernel<128, 128, 64, 4, true, false>(fa::BwdArgs)", ("dkdv", "causal")),
    ("void fa::dkdv_wide_kernel<128, 96, 32, 4, true, true>(fa::BwdArgs)", ("dkdv_atomic", "causal")),
    ("void fa::preprocess_kernel<128>(fa::PreArgs)", ("preprocess", None)),
    # forward with optimistic statistics: <D, DV, tile, waves, occupancy, CAUSAL, DROP, OPT>
    ("void fa::fwd_kernel<128, 128, 32, 4, 3, false, false, true>(fa::FwdArgs)", ("fwd", "full")),
    ("void fa::fwd_kernel<128, 128, 32, 4, 3, true, false, true>(fa::FwdArgs)", ("fwd", "causal")),
    # column-window dK/dV above 256: <D, DV, window, BQ, waves, CAUSAL, ATOMIC>
    ("void fa::dkdv_split_kernel<384, 320, 128, 32, 4, true, true>(fa::BwdArgs)", ("dkdv_atomic", "causal")),
    ("void fa::dkdv_split_kernel<384, 384, 128, 32, 4, false, false>(fa::BwdArgs)", ("dkdv", "full")),
])
def test_classify(name, expected):
    assert classify(name) == expected


@pytest.mark.parametrize("name", [
    # dropout kernels (last template argument true) are timed by their own report
    "void fa::fwd_kernel<128, 128, 64, 4, 2, false, true>(fa::FwdArgs)",
    "void fa::fwd_kernel<128, 128, 64, 4, 2, false, true, false>(fa::FwdArgs)",
    "void fa::dkdv_kernel<128, 128, 64, 4, false, false, 0, false, true>(fa::BwdArgs)",
    "void elementwise_copy_kernel(float*)",
])
def test_classify_skips(name):
    assert classify(name) is None


def _write_csv(path, header, rows):
    import csv
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_profsum_stats_table(tmp_path):
    from exact_attention_102_amd.profsum import stats_table
    d = tmp_path / "prof"
    d.mkdir()
    _write_csv(d / "run_kernel_stats.csv",
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [["void fa::fwd_kernel<128, 128, 32, 4, 3, false, false>(fa::FwdArgs)", 2, 300000, 150000, 25.0,
                 140000, 160000],
                ["void fa::dq_kernel<128, 128, 64, 8, 2, false, false>(fa::BwdArgs)", 2, 900000, 450000, 75.0,
                 440000, 460000]])
    lines = stats_table(str(d)).splitlines()
    # sorted by total time, durations in microseconds / milliseconds
    assert "dq_kernel" in lines[2] and "| 2 | 450.0 | 440.0 | 460.0 | 0.90 | 75.0 |" in lines[2]
    assert "fwd_kernel" in lines[3] and "| 150.0 |" in lines[3]


def test_profsum_sq_table(tmp_path):
    from exact_attention_102_amd.profsum import sq_table
    d = tmp_path / "pmc"
    d.mkdir()
    name = "void fa::fwd_kernel<128, 128, 32, 4, 3, false, false>(fa::FwdArgs)"
    pairs = 4 * 16 * 2048 * 2048  # b4_h16_n2048_d128, non-causal
    rows = [[1, name, "GRBM_GUI_ACTIVE", 8 * 1000.0],
            [1, name, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 400.0],
            [1, name, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e9],
            [1, name, "SQ_INSTS_VALU", pairs * 7 / 64],
            [1, name, "SQ_INSTS_VALU_TRANS_F32", pairs / 64],
            [1, name, "SQ_LDS_IDX_ACTIVE", 100.0],
            [1, name, "SQ_LDS_BANK_CONFLICT", 25.0]]
    _write_csv(d / "run_counter_collection.csv", ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    row = sq_table(str(d), "b4_h16_n2048_d128").splitlines()[2]
    # busy = 400 / 1000 per SIMD; 1e9 MOPS x 512 flop; 7 and 1 lane-ops per score element; 25% conflicts
    assert "| 512.0 | 7.00 | 1.00 | 0.250 |" in row
    cells = [x.strip() for x in row.split("|")]
    assert cells[2] == "40.0"
    # VALU / TRANS busy estimates: instructions x measured issue cycles / (1000 cycles x 1024 SIMDs)
    from exact_attention_102_amd.profsum import MFMA_FLOP, TRANS_CYCLES, VALU_CYCLES
    n_mfma = 512e9 / MFMA_FLOP
    n_valu, n_trans = pairs * 7 / 64, pairs / 64
    want_trans = 100 * n_trans * TRANS_CYCLES / (1000 * 1024)
    want_valu = 100 * ((n_valu - n_mfma - n_trans) * VALU_CYCLES + n_trans * TRANS_CYCLES) / (1000 * 1024)
    assert abs(float(cells[3]) - want_valu) <= 0.05 + 1e-3 * want_valu
    assert abs(float(cells[4]) - want_trans) <= 0.05 + 1e-3 * want_trans
