"""Host-side logic of bench.py (no GPU needed): the one-GPU guard, kernel labels, and the counter
summaries built from rocprofv3 CSV files (synthetic rows here, with known answers)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    sys.path.insert(0, ROOT)
    import bench as b
    return b


def test_more_than_one_gpu_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_kernel_labels(bench):
    lab = bench.kernel_label
    assert lab("void fa::(anonymous namespace)::fwd_bf16_kernel<128, true, false, false>(fa::FwdArgs, fa::Sched)") == "fwd"
    assert lab("void fa::(anonymous namespace)::fwd_bf16_kernel<64, false, true, false>(fa::FwdArgs, fa::Sched)") == \
        "fwd_noncausal"
    assert lab("void fa::(anonymous namespace)::bwd_dkdv_kernel<128, true, false>(fa::BwdArgs, fa::Sched)") == "bwd_dkdv"
    assert lab("void fa::(anonymous namespace)::bwd_dkdv_wave_kernel<64, true, false>(fa::BwdArgs, fa::Sched)") == \
        "bwd_dkdv"
    assert lab("void fa::(anonymous namespace)::fwd_mxfp8_kernel<128, true, false>(fa::Fp8FwdArgs, fa::Sched)") == \
        "fwd_mxfp8"
    assert lab("_ZN2fa12_GLOBAL__N_121mx_quantize_vt_kernelILi128EEEvPKDF16bPhS4_ii") == "mxfp8_quantize_vt"
    assert lab("void fa::(anonymous namespace)::fwd_bf16_kernel<128, true, false, false, 8>(fa::FwdArgs, fa::Sched)") == "fwd"
    assert lab("void fa::(anonymous namespace)::fwd_pingpong_kernel<true>(fa::FwdArgs, fa::Sched)") == "fwd_pingpong"
    assert lab("void fa::(anonymous namespace)::fwd_pingpong_kernel<false>(fa::FwdArgs, fa::Sched)") == \
        "fwd_pingpong_noncausal"
    assert lab("__amd_rocclr_copyBuffer") is None


def _write_counter_csv(path, rows):
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_from_scales_by_the_copy_calibration(bench, tmp_path, monkeypatch):
    # a 256 MiB copy reads 128 MiB on FETCH_SIZE (factor 2) and 256 MiB on WRITE_SIZE (factor 1);
    # the forward's counters in KiB scale by those factors; per-dispatch rows are summed
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "hbm.json"))
    fwd = "void fa::(anonymous namespace)::fwd_bf16_kernel<128, true, false, false>(fa::FwdArgs, fa::Sched)"
    mib = 1024  # KiB
    fetch = [{"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
              "Counter_Value": 128 * mib},
             {"Dispatch_Id": 2, "Kernel_Name": fwd, "Counter_Name": "FETCH_SIZE", "Counter_Value": 100 * mib},
             {"Dispatch_Id": 2, "Kernel_Name": fwd, "Counter_Name": "FETCH_SIZE", "Counter_Value": 50 * mib}]
    write = [{"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE",
              "Counter_Value": 256 * mib},
             {"Dispatch_Id": 2, "Kernel_Name": fwd, "Counter_Name": "WRITE_SIZE", "Counter_Value": 64 * mib}]
    for r in fetch + write:
        r.update(Start_Timestamp=0, End_Timestamp=1000)
    _write_counter_csv(tmp_path / "f.csv", fetch)
    _write_counter_csv(tmp_path / "w.csv", write)
    bench.traffic_from(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), workload="long")
    rec = json.load(open(tmp_path / "hbm.json"))
    assert rec["fetch_size_factor"] == pytest.approx(2.0) and rec["write_size_factor"] == pytest.approx(1.0)
    k = {e["kernel"]: e for e in rec["kernels"]}["fwd"]
    assert k["fetch_bytes_per_launch"] == pytest.approx(2 * 150 * 2 ** 20)
    assert k["write_bytes_per_launch"] == pytest.approx(64 * 2 ** 20)
    assert rec["csrc_sha256"] == bench.csrc_digest()


def test_mfma_from_busy_fraction(bench, tmp_path):
    # 1024 SIMDs x 1000 cycles per XCD (GRBM_GUI_ACTIVE is summed over 8 XCDs) with 512000 busy
    # cycles is 50% busy; 1000 cycles per XCD over 500 ns is a 2 GHz clock
    dkdv = "void fa::(anonymous namespace)::bwd_dkdv_kernel<128, true, false>(fa::BwdArgs, fa::Sched)"
    rows = []
    for name, val in (("SQ_VALU_MFMA_BUSY_CYCLES", 512000), ("GRBM_GUI_ACTIVE", 8000), ("SQ_INSTS_MFMA", 16000)):
        rows.append({"Dispatch_Id": 5, "Kernel_Name": dkdv, "Counter_Name": name, "Counter_Value": val,
                     "Start_Timestamp": 0, "End_Timestamp": 500})
    _write_counter_csv(tmp_path / "m.csv", rows)
    table = bench.mfma_from(str(tmp_path / "m.csv"))
    line = [l for l in table.splitlines() if l.startswith("| bwd_dkdv")][0]
    assert "50.0%" in line and "2.00 GHz" in line


def test_data_sensitivity_from_groups_cases_in_call_order(bench, tmp_path):
    # four forward cases, then four GEMM cases, SENS_CALLS dispatches each; a fill kernel without
    # MFMA instructions in between is ignored.  The first two calls of each case are warm-up.
    fwd = "void fa::(anonymous namespace)::fwd_bf16_kernel<128, true, false, false>(fa::FwdArgs, fa::Sched)"
    gemm = "Cijk_Alik_Bljk_BBS_BH_MT256x256x64"
    n = bench.SENS_CALLS
    rows, dsp = [], 0

    def add(name, busy, mfma):
        nonlocal dsp
        dsp += 1
        for cname, val in (("SQ_VALU_MFMA_BUSY_CYCLES", busy), ("GRBM_GUI_ACTIVE", 8000), ("SQ_INSTS_MFMA", mfma)):
            rows.append({"Dispatch_Id": dsp, "Kernel_Name": name, "Counter_Name": cname, "Counter_Value": val,
                         "Start_Timestamp": 0, "End_Timestamp": 500})

    for case in range(4):
        for i in range(n):
            add(fwd, 1024 * 100 * (case + 1) if i >= 2 else 0, 10)
    add("void at::native::fill_kernel", 0, 0)
    for case in range(4):
        for i in range(n):
            add(gemm, 1024 * 200 * (case + 1) if i >= 2 else 0, 10)
    _write_counter_csv(tmp_path / "s.csv", rows)
    table = bench.data_sensitivity_from(str(tmp_path / "s.csv")).splitlines()
    fwd_lines = [l for l in table if l.startswith("| attention forward")]
    gemm_lines = [l for l in table if l.startswith("| library GEMM")]
    assert len(fwd_lines) == 4 and len(gemm_lines) == 4
    assert "| zeros |" in fwd_lines[2] and "30.0%" in fwd_lines[2] and "2.00" in fwd_lines[2]
    assert "zeros" in gemm_lines[1] and "40.0%" in gemm_lines[1]
    assert all(f"| {n - 2} |" in l for l in fwd_lines + gemm_lines)


def test_percentiles_nearest_rank(bench):
    p = bench.percentiles([5.0, 1.0, 4.0, 2.0, 3.0, 6.0, 7.0, 8.0, 9.0, 10.0, 11.0])
    assert p == {"p10_ms": 2.0, "p50_ms": 6.0, "p90_ms": 10.0}
    assert bench.percentiles([3.0]) == {"p10_ms": 3.0, "p50_ms": 3.0, "p90_ms": 3.0}


def test_counter_summaries_refuse_mixed_kernels(bench, tmp_path):
    # the d = 64 forward of another workload under the same label as the d = 128 one: refused
    rows = []
    for dsp, name in ((1, "void fa::(anonymous namespace)::fwd_bf16_kernel<128, true, false, false>(fa::FwdArgs, fa::Sched)"),
                      (2, "void fa::(anonymous namespace)::fwd_bf16_kernel<64, true, false, false>(fa::FwdArgs, fa::Sched)")):
        for cname, val in (("SQ_VALU_MFMA_BUSY_CYCLES", 1000), ("GRBM_GUI_ACTIVE", 8000), ("SQ_INSTS_MFMA", 10)):
            rows.append({"Dispatch_Id": dsp, "Kernel_Name": name, "Counter_Name": cname, "Counter_Value": val,
                         "Start_Timestamp": 0, "End_Timestamp": 500})
    _write_counter_csv(tmp_path / "m.csv", rows)
    with pytest.raises(SystemExit, match="no-other-workloads"):
        bench.mfma_from(str(tmp_path / "m.csv"))


def test_counters_from_shares_of_wave_cycles(bench, tmp_path):
    # two dispatches of the dK/dV kernel: medians of the per-dispatch sums, wait and active
    # counters also as a share of SQ_WAVE_CYCLES
    name = "void fa::(anonymous namespace)::bwd_dkdv_kernel<128, true, false>(fa::BwdArgs, fa::Sched)"
    rows = []
    for dsp, scale in ((1, 1.0), (2, 1.0)):
        for cname, val in (("SQ_WAVE_CYCLES", 1000.0), ("SQ_WAIT_ANY", 250.0), ("SQ_LDS_BANK_CONFLICT", 0.0)):
            for part in range(2):  # rows of one dispatch are summed
                rows.append({"Dispatch_Id": dsp, "Kernel_Name": name, "Counter_Name": cname,
                             "Counter_Value": val * scale / 2, "Start_Timestamp": 0, "End_Timestamp": 1})
    _write_counter_csv(tmp_path / "c.csv", rows)
    table = bench.counters_from(str(tmp_path / "c.csv")).splitlines()
    assert table[0].startswith("| kernel | dispatches | SQ_LDS_BANK_CONFLICT | SQ_WAIT_ANY | SQ_WAVE_CYCLES |")
    line = [l for l in table if l.startswith("| bwd_dkdv")][0]
    assert "| 2 |" in line and "250 (25.0%)" in line and "| 1000 |" in line


def test_cpu_baseline_pool_joins(bench):
    """The host oracle runs on a process pool (one (b, h) per task) and leaves no child process."""
    import multiprocessing

    import workloads

    w = workloads.Workload("pool", 1, 3, 96, 64, "bf16", True, 77, 0.125, description="pool test")
    t = workloads.make(w, with_do=True)
    r = bench.cpu_baseline(w, t, heads=3)
    assert r["kind"] == "oracle" and r["cores"] >= 1 and r["value"] > 0
    assert "3 of 3 heads" in r["sample"]
    assert multiprocessing.active_children() == []
