"""bench.py's profile summaries (bench.py --profile-workload) from rocprofv3 CSV files, on the
CPU: synthetic kernel-trace and counter-collection files with known values go in, and the
figures of profiles/counters_*.md, profiles/sq_*.md and profiles/copy_calibration.md come out
as computed by hand here (durations, percentiles, calibrated bytes, request-size bytes, VALU
busy), with the records bench.py reads back."""
from __future__ import annotations

import csv
import os

import pytest

import bench
from qk_rmsnorm_rope_amd import workloads as wl

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id",
              "Kernel_Id", "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp",
              "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count",
              "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X",
              "Grid_Size_Y", "Grid_Size_Z"]
PMC_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
            "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
            "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
            "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_csv(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, cols)
        wr.writeheader()
        for r in rows:
            wr.writerow({c: r.get(c, 0) for c in cols})


def pmc(out, pass_name, name, kernel, values, dispatches=3):
    rows = [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": c, "Counter_Value": 1.0}
            for c in values]
    for d in range(dispatches):
        rows += [{"Kernel_Name": kernel, "Dispatch_Id": d, "Counter_Name": c, "Counter_Value": v}
                 for c, v in values.items()]
    write_csv(os.path.join(out, f"{pass_name}_{name}", "x", f"{pass_name}_counter_collection.csv"),
              PMC_COLS, rows)


@pytest.fixture
def root(tmp_path, monkeypatch):
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda w=None: "h" * 16)
    return tmp_path


def test_copy_calibration_summary(root):
    out = str(root / "prof")
    k = "void at::native::vectorized_elementwise_kernel<8, neg>"
    pmc(out, "fetch", "copy", k, {"FETCH_SIZE": 524288.0})
    pmc(out, "write", "copy", k, {"WRITE_SIZE": 1048576.0})
    pmc(out, "rdreq", "copy", k, {"TCC_EA0_RDREQ_sum": 8388608 + 100, "TCC_EA0_RDREQ_128B_sum":
                                  8388608, "TCC_EA0_RDREQ_64B_sum": 100,
                                  "TCC_EA0_RDREQ_32B_sum": 0})
    # kernel trace: 5 warm-up copies of 500 us, then 20 timed ones of 400 and 420 us alternating
    rows, t = [], 0
    for d in [500.0] * 5 + [400.0, 420.0] * 10:
        rows.append({"Kernel_Name": k + "(x)", "Start_Timestamp": t, "End_Timestamp": t + int(d * 1000)})
        rows.append({"Kernel_Name": "__amd_rocclr_fillBuffer", "Start_Timestamp": t + 1,
                     "End_Timestamp": t + 2})
        t += int(d * 1000) + 500
    write_csv(os.path.join(out, "trace_copy", "y", "trace_kernel_trace.csv"), TRACE_COLS, rows)
    path = bench.summarize_copy(out, bench.profile_commands("copy", out))
    text = open(path).read()
    assert bench._record(path, "calibration") == {"fetch_factor": 2.0, "write_factor": 1.0}
    assert "| 8388708 | 8388608 | 100 | 0 | 1,073,748,224 | 1,073,741,824 | 1.00001 |" in text
    # 2 GiB per copy at the timed launches' 410 us average
    gbs = 2 * 2 ** 30 / 410e-6 / 1e9
    assert f"| average duration | 410.00 us |" in text
    assert f"| achieved | {gbs:.0f} GB/s ({100 * gbs / 8000:.1f}% of 8 TB/s) |" in text
    assert "| min / max | 400.00 / 420.00 us |" in text
    assert "--kernel-trace" in text and "--copy-calibration --steps 20 --warmup 5" in text
    assert "bench.py --copy-calibration" in text and str(root) not in text


def test_workload_summary_and_traffic_record(root):
    w = wl.ROPE3D_NEOX_FP8_S18480
    name, out = w.name, str(root / "prof")
    kern = "void qkrope::dev::qkrope_kernel<64, 1, 2, 3, 0, true, 1, true, 2, false>(x)"
    open(root / "profiles" / "copy_calibration.md", "w").write(
        '<!-- calibration {"fetch_factor": 2.0, "write_factor": 1.0} -->')
    # 120 dispatches: 20 of 100 us, then 100 of 70..79 us (the timed replay), 1 us apart
    rows, t = [], 1000
    durs = [100.0] * 20 + [70.0 + (i % 10) for i in range(100)]
    for i, d in enumerate(durs):
        rows.append({"Kernel_Name": kern, "Start_Timestamp": t, "End_Timestamp": t + int(d * 1000),
                     "Workgroup_Size_X": 320, "Grid_Size_X": 5913600, "LDS_Block_Size": 4608,
                     "VGPR_Count": 48})
        rows.append({"Kernel_Name": "__amd_rocclr_fillBuffer", "Start_Timestamp": t + 1,
                     "End_Timestamp": t + 2})
        t += int(d * 1000) + 1000
    write_csv(os.path.join(out, f"trace_{name}", "y", "trace_kernel_trace.csv"), TRACE_COLS, rows)
    read_alg = bench.algorithmic_bytes(w) - bench.output_bytes(w)
    pmc(out, "fetch", name, kern, {"FETCH_SIZE": read_alg / 2048})
    pmc(out, "write", name, kern, {"WRITE_SIZE": bench.output_bytes(w) / 1024,
                                   "TCC_EA0_WRREQ_sum": bench.output_bytes(w) / 64 + 10,
                                   "TCC_EA0_WRREQ_64B_sum": bench.output_bytes(w) / 64})
    pmc(out, "rdreq", name, kern, {"TCC_EA0_RDREQ_sum": read_alg / 128,
                                   "TCC_EA0_RDREQ_128B_sum": read_alg / 128,
                                   "TCC_EA0_RDREQ_64B_sum": 0, "TCC_EA0_RDREQ_32B_sum": 0})
    pmc(out, "sq", name, kern, {"SQ_INSTS_VALU": 92400 * 250.0, "SQ_INSTS_SALU": 92400 * 100.0,
                                "SQ_INSTS_LDS": 92400 * 20.0, "SQ_WAVES": 92400.0,
                                "SQ_ACTIVE_INST_VALU": 0.5 * 256 * 170000,
                                "SQ_LDS_BANK_CONFLICT": 256 * 1700.0,
                                "GRBM_GUI_ACTIVE": 8 * 170000.0})   # summed over 8 XCDs
    write_csv(os.path.join(out, f"sq_{name}", "x", "sq_agent_info.csv"),
              ["Name", "Cu_Count", "Num_Xcc"],
              [{"Name": "AMD EPYC", "Cu_Count": 16, "Num_Xcc": 1},
               {"Name": "gfx950", "Cu_Count": 256, "Num_Xcc": 8}])
    cp, sp = bench.summarize_workload(name, out, bench.profile_commands(name, out))
    rec = bench._record(cp, "traffic")
    avg = sum(durs) / len(durs)
    assert rec["algorithmic_bytes"] == bench.algorithmic_bytes(w)
    assert rec["bytes_per_launch"] == bench.algorithmic_bytes(w)
    assert rec["read_request_bytes"] == read_alg
    assert rec["avg_kernel_us"] == pytest.approx(avg, abs=0.01)
    assert rec["avg_kernel_us_last100"] == pytest.approx(74.5, abs=0.01)
    text = open(cp).read()
    assert "| dispatches | 120 |" in text
    assert "p10 / median / p90 | 71.00 / 75.00 / 79.00 us" in text
    assert "median idle gap between consecutive launches (last 100) | 1.00 us" in text
    assert "| FETCH_SIZE x 2.0 |" in text and "| 1.0000 |" in text
    assert f"{bench.output_bytes(w) // 64:,} of 64 bytes and 10 of 32 bytes" in text
    sq = bench._record(sp, "sq")
    assert sq["valu_per_wave"] == 250.0 and sq["valu_busy_pct"] == 50.0
    assert sq["lds_bank_conflict_per_wave"] == pytest.approx(256 * 1700 / 92400, abs=0.01)
    assert "**50.0%**" in open(sp).read()
    # bench.py reports the record while the hash matches, and not once it differs
    assert bench.traffic_from_profile(w)["bytes_per_launch"] == rec["bytes_per_launch"]
    bench.kernel_source_hash = lambda w=None: "g" * 16
    assert bench.traffic_from_profile(w) is None
