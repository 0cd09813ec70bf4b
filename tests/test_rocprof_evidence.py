"""Host-side checks of the rocprofv3 evidence harness (no GPU, no profiler):
synthetic counter records with known values go through its summaries, and
bench.py reads the traffic figure back."""

import csv
import json
import os

import bench
from exact_masked_scaled_amd import rocprof_evidence as R

FWD = "_ZN4attn10fwd_kernelIDF16bLi128ELi128ELb0ELb0EEEvNS_12KernelParamsE"
DQ = "_ZN4attn13bwd_dq_kernelIDF16bLi128ELi128ELb0ELb0EEEvNS_12KernelParamsE"
DKDV = "_ZN4attn20bwd_dkdv_quad_kernelIDF16bLi128ELi128ELb0ELb0EEEvNS_12KernelParamsE"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float, " \
       "at::native::binary_internal::MulFunctor<float> > >"
FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _records(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _bench_line(raw, name, pairs=1000):
    line = {"value": 1.0, "kernels": {k: {"ms": 1.0} for k in ("fwd", "bwd_dq", "bwd_dkdv")},
            "config": {"visible_pairs": pairs, "d_h": 128, "d_v": 128}}
    with open(os.path.join(raw, f"{name}.out"), "w") as f:
        f.write("progress line\n" + json.dumps(line) + "\n")


def test_traffic_is_scaled_by_the_calibration_copy_and_read_back_by_bench(tmp_path, monkeypatch):
    raw, out = str(tmp_path / "raw"), str(tmp_path / "out")
    gib_kib = R.COPY_MIB * 1024
    # the copy reads half its true bytes on FETCH_SIZE and all of them on WRITE_SIZE
    _records(os.path.join(raw, "fetch"), [
        {"Dispatch_Id": 1, "Kernel_Name": DKDV, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000.0,
         "Start_Timestamp": 0, "End_Timestamp": 10},
        {"Dispatch_Id": 2, "Kernel_Name": DKDV, "Counter_Name": "FETCH_SIZE", "Counter_Value": 3000.0,
         "Start_Timestamp": 0, "End_Timestamp": 10},
        {"Dispatch_Id": 3, "Kernel_Name": COPY, "Counter_Name": "FETCH_SIZE", "Counter_Value": gib_kib / 2,
         "Start_Timestamp": 0, "End_Timestamp": 10},
    ])
    _records(os.path.join(raw, "write"), [
        {"Dispatch_Id": 1, "Kernel_Name": DKDV, "Counter_Name": "WRITE_SIZE", "Counter_Value": 500.0,
         "Start_Timestamp": 0, "End_Timestamp": 10},
        {"Dispatch_Id": 2, "Kernel_Name": COPY, "Counter_Name": "WRITE_SIZE", "Counter_Value": gib_kib,
         "Start_Timestamp": 0, "End_Timestamp": 10},
    ])
    os.makedirs(out)
    R.write_traffic(raw, out)
    path = os.path.join(out, "bwd_dkdv_causal_gqa_b8_n4096_traffic.txt")
    text = open(path).read()
    expect = (2000.0 * 1024) * 2.0 + 500.0 * 1024 * 1.0  # mean FETCH x 2 + WRITE x 1, KiB -> bytes
    assert f"hbm_bytes_per_launch: {expect:.0f}" in text
    assert "fetch_scale: 2.0000" in text and "write_scale: 1.0000" in text
    row = [l for l in text.splitlines() if l.startswith("| `bwd_dkdv_quad_kernel`")][0]
    cells = [c.strip() for c in row.split("|")[2:-1]]
    assert cells[-2] == "0.000" and cells[-1] == f"{expect / 10e-9 / 1e9:.0f}"  # 10 ns dispatches
    monkeypatch.setattr(bench, "TRAFFIC_FILE", path)
    assert bench.load_traffic(None) == expect


def test_traffic_from_other_kernel_sources_is_not_used(tmp_path, monkeypatch):
    path = tmp_path / "t.txt"
    path.write_text("kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.load_traffic(None) is None


def test_mfma_busy_clock_and_wave_shares(tmp_path):
    raw, out = str(tmp_path / "raw"), str(tmp_path / "out")
    # one dK/dV dispatch of 2 ms at 2 GHz: 4e6 cycles per XCD, a quarter of all SIMD cycles busy
    cyc = 4e6
    mf = [("SQ_VALU_MFMA_BUSY_CYCLES", cyc * R.SIMDS / 4), ("SQ_VALU_MFMA_COEXEC_CYCLES", cyc * R.SIMDS / 8),
          ("SQ_INSTS_MFMA", 1000.0), ("SQ_INSTS_VALU", 4000.0), ("SQ_INSTS_LDS", 1500.0),
          ("GRBM_GUI_ACTIVE", cyc * R.XCDS)]
    _records(os.path.join(raw, "mfma"), [
        {"Dispatch_Id": 1, "Kernel_Name": DKDV, "Counter_Name": c, "Counter_Value": v, "Start_Timestamp": 0,
         "End_Timestamp": 2_000_000} for c, v in mf])
    wt = [("SQ_WAVE_CYCLES", 100.0), ("SQ_WAIT_ANY", 30.0), ("SQ_WAIT_INST_ANY", 20.0), ("SQ_ACTIVE_INST_ANY", 50.0),
          ("SQ_ACTIVE_INST_VALU", 25.0), ("SQ_ACTIVE_INST_LDS", 5.0), ("GRBM_GUI_ACTIVE", cyc * R.XCDS)]
    _records(os.path.join(raw, "wait"), [
        {"Dispatch_Id": 1, "Kernel_Name": DKDV, "Counter_Name": c, "Counter_Value": v, "Start_Timestamp": 0,
         "End_Timestamp": 2_000_000} for c, v in wt])
    _bench_line(raw, "mfma", pairs=10**9)
    os.makedirs(out)
    R.write_mfma(raw, out, json.loads(open(os.path.join(raw, "mfma.out")).read().splitlines()[-1]))
    rows = [l for l in open(os.path.join(out, "mfma_utilisation_causal_gqa_b8_n4096.md")) if "bwd_dkdv_quad" in l]
    busy, co, nm, valu, lds, ms, ghz, tf = [c.strip() for c in rows[0].split("|")[2:10]]
    assert busy == "25.0" and co == "50.0" and valu == "3.00" and lds == "1.50"
    assert ms == "2.000" and ghz == "2.00"
    assert tf == f"{2 * 10**9 * 512 / 2e-3 / 1e12:.0f}"  # 2(2d_h + 2d_v) per pair over the dispatch
    busy_any, wait_issue, wait_dep, v_, l_ = [c.strip() for c in rows[1].split("|")[2:7]]
    assert (busy_any, wait_issue, wait_dep, v_, l_) == ("50.0%", "20.0%", "30.0%", "25.0%", "5.0%")


def test_trace_summary_leaves_out_warmups_and_reproduces_the_fraction(tmp_path):
    """The kernel-trace summary drops the benchmark's warm-up dispatches and
    credits the same FLOPs as bench.py, so its fraction for the dominant
    kernel is the bench line's when the durations agree."""
    raw, out = str(tmp_path / "raw"), str(tmp_path / "out")
    os.makedirs(os.path.join(raw, "trace"))
    os.makedirs(out)
    rows = []
    t = 0
    for i in range(R.TRACE_WARMUP + R.TRACE_STEPS):
        for name, dur in ((FWD, 500_000), (DQ, 700_000), (DKDV, 1_000_000)):
            if i < R.TRACE_WARMUP:
                dur *= 3  # slow warm-ups must not count
            rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 1000
    with open(os.path.join(raw, "trace", "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)
    pairs = 10**9
    frac = 2 * pairs * 512 / 1e-3 / 1e12 / bench.PEAK_TFLOPS["bf16"]
    line = {"value": 1.0, "kernels": {k: {"ms": 1.0} for k in ("fwd", "bwd_dq", "bwd_dkdv")},
            "config": {"visible_pairs": pairs, "d_h": 128, "d_v": 128}, "roofline": {"frac": round(frac, 4)}}
    R.write_trace(raw, out, line)
    text = open(os.path.join(out, "kernel_stats_causal_gqa_b8_n4096.md")).read()
    row = [l for l in text.splitlines() if l.startswith("| `bwd_dkdv_quad_kernel`")][0]
    cells = [c.strip() for c in row.split("|")[2:-1]]
    assert cells[0] == str(R.TRACE_STEPS) and cells[1] == "1000.0" and cells[2] == "1000.0"
    assert cells[-1] == f"{frac:.4f}"
    assert f"the trace's {frac:.4f}" in text


def test_recorded_commands_profile_the_committed_benchmark():
    for name in R.PASSES:
        cmd = R.command(name)
        assert cmd.startswith("cd /tmp && export TMPDIR=/tmp && timeout -s KILL ")
        assert "-- python3 $REPO/bench.py " in cmd and "--no-cpu-baseline" in cmd
    # counter passes stay within one rocprofv3 pass's limits (8 SQ, 2 GRBM; byte counters alone)
    for name, (flags, _) in R.PASSES.items():
        names = flags[1:] if flags[0] == "--pmc" else []
        assert sum(n.startswith("SQ_") for n in names) <= 8
        assert sum(n.startswith("GRBM_") for n in names) <= 2
        if any(n in ("FETCH_SIZE", "WRITE_SIZE") for n in names):
            assert len(names) == 1


def test_short_name_mangled_and_demangled():
    """The profiler reports some kernel names mangled, others demangled."""
    assert R.short_name("_ZN4attn15bwd_rows_kernelIDF16bLi128EEEvNS_12KernelParamsE") == "bwd_rows_kernel"
    assert R.short_name("void attn::bwd_dq_gs_kernel<128>(attn::KernelParams)") == "bwd_dq_gs_kernel"
    assert R.short_name("void at::native::elementwise_kernel<128, 2>(int)") is None
