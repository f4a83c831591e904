"""CPU checks of bench.py's counter-record builder (rocprofv3 --pmc CSV passes -> per-kernel
record): calibration scales, clock, busy fractions and HBM bytes on a small synthetic set
of counter files whose expected values follow from the definitions by hand."""

import csv
import json
import os

import pytest

import bench

ATT = "void hstu::(anonymous namespace)::attn_kernel<128, 0, 4, false>(hstu::AttnArgs)"
COPY = "__amd_rocclr_copyBuffer"
DUR_NS = 1_000_000  # 1 ms


def _write(d, name, rows):
    os.makedirs(os.path.join(d, name), exist_ok=True)
    with open(os.path.join(d, name, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for disp, kern, ctr, val in rows:
            w.writerow([disp, kern, ctr, val, 1000, 1000 + DUR_NS])


def test_counter_record_from_synthetic_passes(tmp_path):
    d = str(tmp_path)
    clk_ghz = 2.0
    cycles = clk_ghz * DUR_NS  # shader cycles over the dispatch
    mfma = 1_000_000
    _write(d, "sq1", [(1, ATT, "GRBM_GUI_ACTIVE", 8 * cycles),  # summed over 8 XCDs
                      (1, ATT, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * 1024 * cycles),
                      (1, ATT, "SQ_ACTIVE_INST_VALU", 0.5 * 1024 * cycles / 4),
                      (1, ATT, "SQ_BUSY_CYCLES", 32 * cycles),
                      (1, ATT, "SQ_INSTS_MFMA", mfma)])
    _write(d, "sq2", [(1, ATT, "SQ_INSTS_VALU", 7 * mfma), (1, ATT, "SQ_INSTS_VALU_TRANS_F32", 2 * mfma),
                      (1, ATT, "SQ_INSTS_SALU", 3 * mfma), (1, ATT, "SQ_INSTS_LDS", 1.5 * mfma),
                      (1, ATT, "SQ_LDS_BANK_CONFLICT", 10), (1, ATT, "SQ_ACTIVE_INST_LDS", 100)])
    _write(d, "fetch", [(1, ATT, "FETCH_SIZE", 300_000)])
    _write(d, "write", [(1, ATT, "WRITE_SIZE", 100_000)])
    copy = 1 << 30
    _write(d, "cfetch", [(1, COPY, "FETCH_SIZE", copy / 1024 / 2)])  # reads half: scale 2
    _write(d, "cwrite", [(1, COPY, "WRITE_SIZE", copy / 1024)])       # exact: scale 1
    out = os.path.join(d, "rec.json")
    bench.write_counter_record(d, copy, out_path=out)
    rec = json.load(open(out))
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    a = rec["kernels"]["attention"]
    assert a["ms"] == pytest.approx(1.0)
    assert a["clock_ghz"] == pytest.approx(clk_ghz)
    assert a["mfma_busy_frac"] == pytest.approx(0.25)
    assert a["valu_busy_frac"] == pytest.approx(0.5)
    assert a["sq_busy_frac"] == pytest.approx(1.0)
    assert a["valu_per_mfma"] == pytest.approx(6.0)  # VALU instructions beside the MFMAs
    assert a["trans_per_mfma"] == pytest.approx(2.0)
    assert a["lds_bank_conflict_frac"] == pytest.approx(0.1)
    assert a["fetch_bytes"] == pytest.approx(300_000 * 1024 * 2.0)
    assert a["write_bytes"] == pytest.approx(100_000 * 1024)
    assert a["hbm_gbs"] == pytest.approx((300_000 * 2048 + 100_000 * 1024) / DUR_NS)
    assert a["tflops"] == pytest.approx(a["useful_flops"] / DUR_NS / 1e3)
    assert a["peak_tflops_at_clock"] == pytest.approx(256 * 4 * 1024 * clk_ghz / 1e3)
    assert rec["kernel_sources_sha256"] == bench._kernel_sources_sha()
    # kernels without counter rows are left out
    assert set(rec["kernels"]) == {"attention"}
