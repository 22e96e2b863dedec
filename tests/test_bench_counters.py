"""bench.py's counter parsing (host only): the clock and MFMA-busy figures it
quotes next to the roofline come from one rocprofv3 pass of GRBM_GUI_ACTIVE
and SQ_VALU_MFMA_BUSY_CYCLES."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow({k: r.get(k, 0) for k in FIELDS})


def _dispatch(did, name, ns, gui, mfma):
    base = {"Dispatch_Id": did, "Kernel_Name": name, "Start_Timestamp": 1000,
            "End_Timestamp": 1000 + ns}
    return [dict(base, Counter_Name="GRBM_GUI_ACTIVE", Counter_Value=gui),
            dict(base, Counter_Name="SQ_VALU_MFMA_BUSY_CYCLES", Counter_Value=mfma),
            dict(base, Counter_Name="SQ_BUSY_CYCLES", Counter_Value=1)]


@pytest.mark.parametrize("ghz,busy", [(1.5, 0.75), (2.4, 1.0), (1.9, 0.3)])
def test_clock_counters(tmp_path, ghz, busy):
    ns = 2_000_000                      # a 2 ms dispatch
    cycles = ghz * ns                   # per XCD
    gui = cycles * bench.XCDS           # rocprofv3 sums the XCDs
    mfma = busy * cycles * bench.SIMDS
    name = "void orca::gemm_w4_kernel<1, 4>(orca::bf16 const*)"
    rows = _dispatch(1, name, ns, gui, mfma) + _dispatch(2, name, ns, gui, mfma)
    # a short kernel is left out; other kernels are not GEMM launches
    rows += _dispatch(3, "void orca::tail_reduce_kernel<1, 256>(float const*)", 50_000, 1e9, 0)
    rows += _dispatch(4, "void orca::attn_split_kernel<orca::bf16, 128>(orca::AttnArgs)", ns,
                      gui, 0)
    path = tmp_path / "run_counter_collection.csv"
    _write(path, rows)
    out = bench.clock_counters(str(path))
    assert list(out) == ["orca::gemm_w4_kernel<1, 4>"]
    rec = out["orca::gemm_w4_kernel<1, 4>"]
    assert rec["clock_ghz"] == pytest.approx(ghz, abs=1e-3)
    assert rec["mfma_busy_percent"] == pytest.approx(100 * busy, abs=0.05)
    # 1024 SIMDs x 1024 FLOP per clock: 2.5 PFLOP/s at 2.4 GHz (the published peak)
    assert rec["mfma_ceiling_tflops_at_clock"] == pytest.approx(ghz * 1048.576, abs=0.1)


def test_clock_counters_missing_file(tmp_path):
    assert bench.clock_counters(str(tmp_path / "absent.csv")) == {}
