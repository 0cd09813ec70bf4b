"""rocprofv3 evidence for the benchmark's headline workload.

    python -m exact_masked_scaled_amd.rocprof_evidence [--out profiles] [--raw DIR] [--only PASS ...]

Runs ``bench.py`` (headline workload only, no CPU baseline) under rocprofv3
once per pass and writes three short summaries into ``--out``:

* ``kernel_stats_causal_gqa_b8_n4096.md``: per-kernel time (kernel trace);
* ``bwd_dkdv_causal_gqa_b8_n4096_traffic.txt``: HBM bytes per launch from
  FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter reads for a
  plain 1 GiB copy timed in the same run (bench.py reads the dK/dV figure back,
  keyed by a hash of the kernel sources);
* ``mfma_utilisation_causal_gqa_b8_n4096.md``: MFMA busy cycles over the SIMD
  cycles of each dispatch, VALU/MFMA co-issue, instructions per MFMA, the clock
  of the dispatch, and where the waves' time goes.

Each pass is a child process (``timeout -s KILL`` around ``rocprofv3 ... --
python3 bench.py``) started from /tmp; this process never touches the GPU.
Raw CSV output goes to ``--raw`` (default /tmp/attn_rocprof; the summaries
write it as $RAW).  Counter passes stay within one rocprofv3 pass's hardware
limits (at most 8 SQ and 2 GRBM counters; FETCH_SIZE and WRITE_SIZE in runs of
their own).
"""

from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

# the trace pass times exactly what the default benchmark line times (its
# step and warm-up counts), so the trace reproduces the line's roofline
TRACE_STEPS, TRACE_WARMUP = 20, 5
BENCH_ARGS_TRACE = ["--steps", str(TRACE_STEPS), "--warmup", str(TRACE_WARMUP), "--no-cpu-baseline",
                    "--no-other-workloads"]
BENCH_ARGS_PMC = ["--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--no-other-workloads"]
COPY_MIB = 1024

PASSES = {
    "trace": (["--kernel-trace", "--stats"], BENCH_ARGS_TRACE),
    "fetch": (["--pmc", "FETCH_SIZE"], BENCH_ARGS_PMC + ["--calibrate-copy-mib", str(COPY_MIB)]),
    "write": (["--pmc", "WRITE_SIZE"], BENCH_ARGS_PMC + ["--calibrate-copy-mib", str(COPY_MIB)]),
    "mfma": (["--pmc", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
              "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"], BENCH_ARGS_PMC),
    "wait": (["--pmc", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
              "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "GRBM_GUI_ACTIVE"], BENCH_ARGS_PMC),
}
# the kernels of a step, by the names bench.py reports them under (the
# two-pass backward's dQ pass, or with G_S kept the per-row pass and the G_Q
# product)
KERNELS = {"fwd_kernel": "fwd", "bwd_dq_kernel": "bwd_dq", "bwd_rows_kernel": "bwd_rows",
           "bwd_dkdv_quad_kernel": "bwd_dkdv", "bwd_dq_gs_kernel": "bwd_dq_gs"}
SIMDS, XCDS = 1024, 8  # MI355X: 256 CUs x 4 SIMDs, 8 XCDs
WORKLOAD = "causal GQA bf16, B=8 H_q=32 H_kv=8 n=4096 d=128, padded lengths (seed 1003)"


def short_name(name: str):
    """The kernel's name without namespace and template arguments; the
    profiler reports some names mangled and others demangled."""
    m = re.match(r"_ZN4attn\d+(\w+?)I", name) or re.search(r"attn::(\w+)<", name)
    return m.group(1) if m else None


def command(name: str, repo: str = "$REPO", raw: str = "$RAW") -> str:
    flags, args = PASSES[name]
    lim = "timeout -s KILL 300 " if name == "trace" else "timeout -s KILL 120 "
    return (f"cd /tmp && export TMPDIR=/tmp && {lim}rocprofv3 {' '.join(flags)} -d {raw}/{name} -o run "
            f"--output-format csv -- python3 {repo}/bench.py {' '.join(args)}")


def run_pass(name: str, raw: str) -> dict:
    """One rocprofv3 pass; returns the bench JSON line it printed."""
    flags, args = PASSES[name]
    outdir = os.path.join(raw, name)
    os.makedirs(outdir, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    lim = "300" if name == "trace" else "120"
    cmd = ["timeout", "-s", "KILL", lim, "rocprofv3", *flags, "-d", outdir, "-o", "run", "--output-format", "csv",
           "--", sys.executable, os.path.join(ROOT, "bench.py"), *args]
    print(f"[rocprof_evidence] pass {name}: {' '.join(cmd)}", flush=True)
    res = subprocess.run(cmd, cwd="/tmp", env=env, capture_output=True, text=True)
    with open(os.path.join(raw, f"{name}.out"), "w") as f:
        f.write(res.stdout)
    with open(os.path.join(raw, f"{name}.err"), "w") as f:
        f.write(res.stderr)
    lines = [l for l in res.stdout.splitlines() if l.startswith("{")]
    if res.returncode != 0 and not lines:
        raise RuntimeError(f"pass {name} failed ({res.returncode}); see {raw}/{name}.err")
    print(f"[rocprof_evidence] pass {name}: done (rc {res.returncode})", flush=True)
    return json.loads(lines[-1])


def counters(raw: str, name: str):
    """Per kernel: counter -> list of per-dispatch values, plus dispatch durations (s)."""
    path = os.path.join(raw, name, "run_counter_collection.csv")
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    seen = set()
    with open(path) as f:
        for r in csv.DictReader(f):
            k = short_name(r["Kernel_Name"]) or r["Kernel_Name"]
            agg[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            if r["Dispatch_Id"] not in seen:
                seen.add(r["Dispatch_Id"])
                agg[k]["_dur"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    return agg


def mean(v):
    return sum(v) / len(v)


def trace_durations(raw: str) -> dict:
    """Per kernel of a step: the durations (s) of its timed dispatches, in
    launch order, from the kernel trace (the first TRACE_WARMUP dispatches of
    each kernel are the benchmark's warm-up steps and are left out)."""
    per = collections.defaultdict(list)
    with open(os.path.join(raw, "trace", "run_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            n = short_name(r["Kernel_Name"])
            if n in KERNELS:
                per[n].append((int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9))
    return {n: [d for _, d in sorted(v)][TRACE_WARMUP:] for n, v in per.items()}


def credited_flops(bench: dict) -> dict:
    """Algorithmic FLOPs a launch of each kernel is credited with (as bench.py):
    visible pairs only; the dQ pass gets the G_Q product alone."""
    P = bench["config"]["visible_pairs"]
    dh, dv = bench["config"]["d_h"], bench["config"]["d_v"]
    return {"fwd": 2 * P * (dh + dv), "bwd_dq": 2 * P * dh, "bwd_rows": 0, "bwd_dkdv": 2 * P * (2 * dh + 2 * dv),
            "bwd_dq_gs": 2 * P * dh}


def write_trace(raw: str, out: str, bench: dict):
    sys.path.insert(0, ROOT)
    import bench as B  # noqa: E402  (peak and dominant kernel as the benchmark reports them)

    durs = trace_durations(raw)
    alg = credited_flops(bench)
    peak = B.PEAK_TFLOPS["bf16"]
    o = [f"# Kernel time: {WORKLOAD}\n",
         "Made by `python -m exact_masked_scaled_amd.rocprof_evidence --raw $RAW` (pass `trace`); the command, from the",
         "repository root (`REPO=$PWD`, one MI355X; `RAW` the raw-output directory):\n", "```", command("trace"), "```\n",
         f"Per-dispatch durations from the kernel trace (`run_kernel_trace.csv`); the first {TRACE_WARMUP} dispatches of "
         f"each kernel are the benchmark's warm-up steps and are left out, so the {TRACE_STEPS} dispatches summarised are "
         "the steps the bench line times. Credited TFLOP/s counts visible (query, key) pairs only (forward 2(d_h + d_v), "
         "dQ pass 2 d_h, dK/dV pass 2(2 d_h + 2 d_v), the dQ product from stored score gradients 2 d_h, the per-row "
         "pass 0 FLOP per pair) over the mean duration; fraction of the "
         f"{peak:.0f} TFLOP/s dense bf16 peak.\n",
         "| kernel | timed dispatches | mean (us) | median (us) | min (us) | max (us) | credited TFLOP/s | frac of peak |",
         "|---|---|---|---|---|---|---|---|"]
    fr = {}
    for k, s in KERNELS.items():
        d = durs.get(k)
        if not d:
            continue
        m = mean(d)
        srt = sorted(d)
        med = srt[len(srt) // 2] if len(srt) % 2 else 0.5 * (srt[len(srt) // 2 - 1] + srt[len(srt) // 2])
        fr[s] = alg[s] / m / 1e12 / peak
        o.append(f"| `{k}` | {len(d)} | {m * 1e6:.1f} | {med * 1e6:.1f} | {srt[0] * 1e6:.1f} | {srt[-1] * 1e6:.1f} | "
                 f"{alg[s] / m / 1e12:.1f} | {fr[s]:.4f} |")
    k = bench["kernels"]
    o.append("")
    dom = B.DOMINANT
    line = bench.get("roofline", {}).get("frac")
    o.append(f"The same run's bench line (HIP events on the launch stream, {TRACE_STEPS} timed steps) reported "
             + ", ".join(f"{n} {v['ms']:.3f} ms" for n, v in k.items()) + " and "
             f"{bench['value']:.2f} TFLOP/s for the whole step under the profiler"
             + (f"; its roofline fraction for {dom} was {line:.4f}, the trace's {fr.get(dom, float('nan')):.4f}."
                if line is not None else "."))
    with open(os.path.join(out, "kernel_stats_causal_gqa_b8_n4096.md"), "w") as f:
        f.write("\n".join(o) + "\n")


def write_traffic(raw: str, out: str):
    sys.path.insert(0, ROOT)
    import bench as B  # noqa: E402  (the source hash bench.py checks the figures against)

    fe, wr = counters(raw, "fetch"), counters(raw, "write")
    copy_bytes = COPY_MIB * (1 << 20)
    # the calibration copy: torch's elementwise multiply kernel, three launches
    cf = [v for k, d in fe.items() if "MulFunctor" in k for v in d["FETCH_SIZE"]]
    cw = [v for k, d in wr.items() if "MulFunctor" in k for v in d["WRITE_SIZE"]]
    if not cf or not cw:
        raise RuntimeError("calibration copy not found in the counter records")
    # counters are KiB per dispatch
    fs = copy_bytes / (mean(cf) * 1024)
    ws = copy_bytes / (mean(cw) * 1024)
    o = [f"# HBM traffic per launch: {WORKLOAD}\n",
         "Made by `python -m exact_masked_scaled_amd.rocprof_evidence --raw $RAW` (passes `fetch`, `write`); the commands,",
         "from the repository root (`REPO=$PWD`, one MI355X; `RAW` the raw-output directory), one counter per run:\n", "```", command("fetch"), command("write"),
         "```\n",
         f"Counters are KiB per dispatch. Calibration: a plain elementwise copy of {COPY_MIB} MiB (reads and writes "
         f"{copy_bytes / 1e6:.1f} MB) reads FETCH_SIZE = {mean(cf) * 1024 / 1e6:.1f} MB and WRITE_SIZE = "
         f"{mean(cw) * 1024 / 1e6:.1f} MB, so FETCH_SIZE is scaled by {fs:.3f} and WRITE_SIZE by {ws:.3f}. Each figure is "
         "the mean over the launches of the run; HBM GB/s divides the calibrated bytes by the mean duration of the "
         "same dispatches (their start and end timestamps in the counter records), against the 8 TB/s peak.\n",
         "| kernel | FETCH_SIZE raw (MB) | WRITE_SIZE raw (MB) | HBM read (MB) | HBM write (MB) | total (MB) | "
         "dispatch (ms) | HBM GB/s |",
         "|---|---|---|---|---|---|---|---|"]
    dom = None
    for k in KERNELS:
        if k not in fe or k not in wr:
            continue
        f_ = mean(fe[k]["FETCH_SIZE"]) * 1024
        w_ = mean(wr[k]["WRITE_SIZE"]) * 1024
        tot = f_ * fs + w_ * ws
        dur = mean(fe[k]["_dur"] + wr[k]["_dur"])  # the dispatches of both passes
        o.append(f"| `{k}` | {f_ / 1e6:.1f} | {w_ / 1e6:.1f} | {f_ * fs / 1e6:.1f} | {w_ * ws / 1e6:.1f} | {tot / 1e6:.1f} | "
                 f"{dur * 1e3:.3f} | {tot / dur / 1e9:.0f} |")
        if KERNELS[k] == B.DOMINANT:
            dom = tot
    if dom is None:
        raise RuntimeError("no counter records for the dominant kernel")
    o += ["", f"Machine-readable figures for the dominant kernel ({B.DOMINANT}), read by bench.py; the hash is over the",
          f"kernel sources the figures were taken with ({', '.join(B.KERNEL_SOURCES)}):\n",
          f"kernel_source_sha256_16: {B.kernel_source_hash()}", f"hbm_bytes_per_launch: {dom:.0f}",
          f"fetch_scale: {fs:.4f}", f"write_scale: {ws:.4f}"]
    with open(os.path.join(out, "bwd_dkdv_causal_gqa_b8_n4096_traffic.txt"), "w") as f:
        f.write("\n".join(o) + "\n")


def write_mfma(raw: str, out: str, bench: dict):
    A, Wt = counters(raw, "mfma"), counters(raw, "wait")
    P = bench["config"]["visible_pairs"]
    dh, dv = bench["config"]["d_h"], bench["config"]["d_v"]
    executed = {"fwd": 2 * P * (dh + dv), "bwd_dq": 2 * P * (2 * dh + dv), "bwd_rows": 0,
                "bwd_dkdv": 2 * P * (2 * dh + 2 * dv), "bwd_dq_gs": 2 * P * dh}
    o = [f"# MFMA utilisation and wave-time breakdown: {WORKLOAD}\n",
         "Made by `python -m exact_masked_scaled_amd.rocprof_evidence --raw $RAW` (passes `mfma`, `wait`); the commands,",
         "from the repository root (`REPO=$PWD`, one MI355X; `RAW` the raw-output directory):\n", "```", command("mfma"), command("wait"), "```\n",
         "rocprofv3 sums each counter over the chip (GRBM_GUI_ACTIVE over the 8 XCDs, so one XCD's active cycles are an",
         "eighth of it); figures are means over the launches of a pass. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /",
         "(GRBM_GUI_ACTIVE / 8 x 1024 SIMDs). The clock is one XCD's GRBM_GUI_ACTIVE cycles over the dispatch's own",
         "duration (its start and end timestamps in the same record); the published 2.5 PFLOP/s dense bf16 peak assumes",
         "2.4 GHz, so at the measured clock the matrix cores deliver at most clock / 2.4 GHz of it.\n",
         "| kernel | MFMA busy (% of SIMD cycles) | VALU issued while MFMA busy (% of MFMA busy) | MFMA instr | other VALU "
         "instr per MFMA | LDS instr per MFMA | dispatch (ms) | clock (GHz) | executed MFMA TFLOP/s |",
         "|---|---|---|---|---|---|---|---|---|"]
    for k, s in KERNELS.items():
        if k not in A:
            continue
        a = {c: mean(v) for c, v in A[k].items()}
        if a["SQ_INSTS_MFMA"] == 0:  # the per-row pass has no products
            continue
        act = a["GRBM_GUI_ACTIVE"] / XCDS
        busy = a["SQ_VALU_MFMA_BUSY_CYCLES"] / (act * SIMDS)
        co = a["SQ_VALU_MFMA_COEXEC_CYCLES"] / a["SQ_VALU_MFMA_BUSY_CYCLES"]
        nm = a["SQ_INSTS_MFMA"]
        dur = a["_dur"]
        o.append(f"| `{k}` | {100 * busy:.1f} | {100 * co:.1f} | {nm:.3g} | {(a['SQ_INSTS_VALU'] - nm) / nm:.2f} | "
                 f"{a['SQ_INSTS_LDS'] / nm:.2f} | {dur * 1e3:.3f} | {act / dur / 1e9:.2f} | "
                 f"{executed[s] / dur / 1e12:.0f} |")
    o += ["", "Where each wave's time goes (SQ_* wave-cycle counters, units of 4 cycles, as a share of SQ_WAVE_CYCLES):\n",
          "| kernel | issuing any instruction | waiting to issue (unit or SIMD busy) | waiting on a dependency (waitcnt, "
          "barrier) | of which VALU issue | of which LDS issue |", "|---|---|---|---|---|---|"]
    for k in KERNELS:
        if k not in Wt:
            continue
        w = {c: mean(v) for c, v in Wt[k].items()}
        t = w["SQ_WAVE_CYCLES"]
        o.append(f"| `{k}` | {100 * w['SQ_ACTIVE_INST_ANY'] / t:.1f}% | {100 * w['SQ_WAIT_INST_ANY'] / t:.1f}% | "
                 f"{100 * w['SQ_WAIT_ANY'] / t:.1f}% | {100 * w['SQ_ACTIVE_INST_VALU'] / t:.1f}% | "
                 f"{100 * w['SQ_ACTIVE_INST_LDS'] / t:.1f}% |")
    o += ["", "Executed MFMA work per visible pair: forward 2(d_h + d_v), dQ pass 2(2d_h + d_v) (it recomputes S and dP), "
          "dK/dV pass 2(2d_h + 2d_v), dQ product from stored score gradients 2d_h FLOP (the per-row pass has none)."]
    with open(os.path.join(out, "mfma_utilisation_causal_gqa_b8_n4096.md"), "w") as f:
        f.write("\n".join(o) + "\n")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--raw", default="/tmp/attn_rocprof")
    ap.add_argument("--only", nargs="*", choices=["trace", "traffic", "mfma"], default=None,
                    help="summaries to (re)make; default all")
    ap.add_argument("--no-run", action="store_true", help="only summarise the raw output of earlier passes")
    a = ap.parse_args(argv)
    a.raw = os.path.abspath(a.raw)  # the passes run from /tmp
    a.out = os.path.abspath(a.out)
    want = set(a.only or ["trace", "traffic", "mfma"])
    need = {"trace": ["trace"], "traffic": ["fetch", "write"], "mfma": ["mfma", "wait"]}
    os.makedirs(a.raw, exist_ok=True)
    os.makedirs(a.out, exist_ok=True)
    benches = {}
    for w in ("trace", "traffic", "mfma"):
        if w not in want:
            continue
        for p in need[w]:
            if a.no_run:
                with open(os.path.join(a.raw, f"{p}.out")) as f:
                    benches[p] = json.loads([l for l in f.read().splitlines() if l.startswith("{")][-1])
            else:
                benches[p] = run_pass(p, a.raw)
    if "trace" in want:
        write_trace(a.raw, a.out, benches["trace"])
    if "traffic" in want:
        write_traffic(a.raw, a.out)
    if "mfma" in want:
        write_mfma(a.raw, a.out, benches["mfma"])
    print(f"[rocprof_evidence] summaries written to {a.out}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
