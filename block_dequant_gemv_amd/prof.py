"""Summaries of rocprofv3 CSV output for this library's kernels.

    python -m block_dequant_gemv_amd.prof trace  <dir> [--skip N] [--tail N]   # --kernel-trace --stats -f csv
    python -m block_dequant_gemv_amd.prof counters <dir> [traffic.json]
    python -m block_dequant_gemv_amd.prof collect <out_dir> [--only trace_step,trace_calls,traffic,sq,trace_gemm,gemm_sq]
    python -m block_dequant_gemv_amd.prof traffic <fetch_dir> <write_dir> [--json out.json]
                                              [--call LABEL=KERNEL|WORKGROUPSxWG ...]

`trace` groups the dispatches by kernel name and grid size (two calls of one
kernel template with different shapes, e.g. the fused QKV and the LM head, show
up as separate rows) and prints count, mean / median / min duration; --skip N
leaves out the first N dispatches of every shape, --tail N keeps only the last N
(the headline's back-to-back roofline batch, which bench.py runs last).

`counters` reads one counter run (--pmc with any counters, plus --kernel-trace)
and prints, per launch shape, the mean of every counter and of the dispatch
time; with GRBM_GUI_ACTIVE it derives the shader clock (busy cycles per
microsecond of dispatch), with SQ_WAVES and SQ_INSTS_VALU the VALU instructions
per wavefront. Given the HBM bytes per dispatch of a traffic run (its
traffic.json, or the same `collect`), it adds each launch shape's HBM rate over
this run's dispatch time and HBM bytes per shader clock.

`collect` runs the profiler passes behind profiles/ (each rocprofv3 pass a
child process of its own under `timeout -s KILL`, the program after `--`):
  trace_step   --kernel-trace --stats of the headline decode step alone
               (bench.py --no-configs --no-cpu --no-q8-step --no-graph)
  trace_calls  --kernel-trace --stats of the per-call table, cold calls only
               (bench.py --no-cpu --no-graph --no-warm)
  fetch, write --pmc FETCH_SIZE / WRITE_SIZE of the headline step and the
               configurations' calls (bench.py ... --calib-copy)
  sq           --pmc SQ_WAVES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_BUSY_CYCLES
               SQ_INSTS_LDS GRBM_GUI_ACTIVE --kernel-trace, same calls
  trace_gemm   --kernel-trace --stats of the prefill GEMM rows
               (bench.py --no-cpu --no-graph --no-q8-step --only "g ")
  gemm_sq      --pmc SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES
               SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_SALU SQ_INSTS_LDS GRBM_GUI_ACTIVE
               --kernel-trace, the same GEMM rows
and writes <out>/*.txt summaries that start with the command that made them.

`traffic` reads two counter runs (--pmc FETCH_SIZE, then --pmc WRITE_SIZE; the
counters are KiB per dispatch) and prints the mean per launch shape. The bytes
are scaled by the factor that makes a plain copy-like kernel of known traffic
read and write exactly its size: `bench.py --calib-copy` runs torch.neg over a
256 MiB buffer (256 MiB read, 256 MiB written per dispatch).
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import statistics as st
import sys
from collections import defaultdict

CALIB_BYTES = 256 << 20
XCDS = 8        # MI355X: accelerator complex dies, each with its own GRBM
SIMDS = 1024    # 256 CUs x 4 SIMDs
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


GEMV_SOURCES = ("layout.h", "dequant.h", "qgemv_kernels.h", "qgemv_device.h", "qgemv_inst.hip",
                "qgemv_kernels.hip", "qgemv_api.hip")


def kernel_source_hash() -> str:
    """Hash of the GEMV path's sources (kernels, layout, launch planning); the counter
    results of its kernels are only valid for the sources they were taken on."""
    h = hashlib.sha256()
    for p in [os.path.join(CSRC, n) for n in GEMV_SOURCES]:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _rows(path_glob: str):
    out = []
    for p in sorted(glob.glob(path_glob, recursive=True)):
        with open(p, newline="") as f:
            out += list(csv.DictReader(f))
    return out


def _get(row: dict, *names, default=None):
    low = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in low and low[n.lower()] not in (None, ""):
            return low[n.lower()]
    return default


def _grid(row) -> int:
    g = _get(row, "Grid_Size_X", "Grid_Size", "grid_size_x", default="0")
    return int(float(g))


def _wg(row) -> int:
    g = _get(row, "Workgroup_Size_X", "Workgroup_Size", default="1")
    return max(1, int(float(g)))


def _short(name: str) -> str:
    name = name.replace("void ", "")
    cut = name.find("(")
    return name[:cut] if cut > 0 else name


def trace_summary(directory: str, skip: int = 0, tail: int = 0, stats_csv: bool = True) -> str:
    """Per launch shape, in dispatch order: count, mean / median / min duration;
    with skip > 0 the first `skip` dispatches of every shape (warm-up) are left
    out; with tail > 0 only the last `tail` dispatches of every shape are kept."""
    rows = _rows(os.path.join(directory, "**", "*kernel_trace.csv"))
    groups = defaultdict(list)
    for r in rows:
        name = _short(_get(r, "Kernel_Name", default="?"))
        t0 = int(_get(r, "Start_Timestamp", default="0"))
        t1 = int(_get(r, "End_Timestamp", default="0"))
        groups[(name, _grid(r) // _wg(r), _wg(r))].append((t0, (t1 - t0) / 1e3))
    groups = {k: [d for _, d in sorted(v)][skip:] for k, v in groups.items()}
    if tail > 0:
        groups = {k: v[-tail:] for k, v in groups.items()}
    groups = {k: v for k, v in groups.items() if v}
    lines = ([f"the first {skip} dispatches of every launch shape left out"] if skip else []) + \
        ([f"the last {tail} dispatches of every launch shape only"] if tail else []) + \
        [f"{'kernel':58s} {'workgroups':>10s} {'wg':>4s} {'n':>5s} {'mean_us':>9s} {'median_us':>9s} "
         f"{'min_us':>8s} {'total_us':>10s}"]
    for (name, wgs, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{name[:58]:58s} {wgs:10d} {wg:4d} {len(d):5d} {st.mean(d):9.2f} {st.median(d):9.2f} "
                     f"{min(d):8.2f} {sum(d):10.1f}")
    stats = _rows(os.path.join(directory, "**", "*kernel_stats.csv")) if stats_csv else []
    if stats:
        lines.append("")
        lines.append("rocprofv3 kernel_stats.csv (per kernel name):")
        keys = list(stats[0].keys())
        lines.append(",".join(keys))
        for r in stats:
            lines.append(",".join(str(r[k]) for k in keys))
    return "\n".join(lines)


def _counter_means(directory: str, counter: str):
    rows = _rows(os.path.join(directory, "**", "*counter_collection.csv"))
    groups = defaultdict(list)
    for r in rows:
        if _get(r, "Counter_Name", default="") != counter:
            continue
        name = _short(_get(r, "Kernel_Name", default="?"))
        groups[(name, _grid(r) // _wg(r), _wg(r))].append(float(_get(r, "Counter_Value", default="0")) * 1024.0)
    return {k: st.mean(v) for k, v in groups.items()}, {k: len(v) for k, v in groups.items()}


def shape_bytes(traffic: dict) -> dict:
    """(kernel, workgroups, workgroup size) -> HBM bytes per dispatch (fetch + write) of a
    traffic summary's data (traffic_summary's second result, or its traffic.json)."""
    out = {}
    for key, v in traffic.get("kernels", {}).items():
        name, shape = key.rsplit("|", 1)
        wgs, wg = (int(t) for t in shape.split("x"))
        out[(name, wgs, wg)] = v["fetch_bytes"] + v["write_bytes"]
    return out


def counter_summary(directory: str, hbm_bytes: dict | None = None) -> str:
    rows = _rows(os.path.join(directory, "**", "*counter_collection.csv"))
    vals = defaultdict(lambda: defaultdict(list))
    durs = defaultdict(dict)
    names = set()
    for r in rows:
        key = (_short(_get(r, "Kernel_Name", default="?")), _grid(r) // _wg(r), _wg(r))
        c = _get(r, "Counter_Name", default="")
        names.add(c)
        vals[key][c].append(float(_get(r, "Counter_Value", default="0")))
        t0, t1 = _get(r, "Start_Timestamp"), _get(r, "End_Timestamp")
        did = _get(r, "Dispatch_Id", "Correlation_Id", default=None)
        if t0 is not None and t1 is not None and did is not None:
            durs[key][did] = (int(t1) - int(t0)) / 1e3
    cols = sorted(names)
    lines = ["per launch shape: dispatches, mean dispatch time (us), mean of each counter per dispatch (rocprofv3 sums "
             "each counter over the device's 8 XCDs)"
             + (";\nclock_MHz = GRBM_GUI_ACTIVE / 8 XCDs / dispatch time (the counter also runs for a few us around "
                "the dispatch, so short kernels read high)" if "GRBM_GUI_ACTIVE" in names else "")
             + (";\nvalu_per_wave = SQ_INSTS_VALU / SQ_WAVES" if {"SQ_WAVES", "SQ_INSTS_VALU"} <= names else "")
             + (";\nvalu_busy = SQ_INSTS_VALU x 4 cycles (a wave64 instruction on a 16-lane SIMD) / (1024 SIMDs x "
                "GRBM_GUI_ACTIVE / 8)" if {"GRBM_GUI_ACTIVE", "SQ_INSTS_VALU"} <= names else "")
             + (";\nmfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8); valu_per_mfma = "
                "(SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA (SQ_INSTS_VALU counts the MFMA instructions too); "
                "coexec = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES"
                if {"GRBM_GUI_ACTIVE", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES"} <= names else "")
             + (";\nhbm_GBps, hbm_B_per_clk = the launch shape's HBM bytes per dispatch from the traffic run (FETCH_SIZE "
                "+ WRITE_SIZE, calibrated) over this run's dispatch time and over its GRBM_GUI_ACTIVE / 8 shader clocks "
                "(the profiler serialises the dispatches of both runs)" if hbm_bytes and "GRBM_GUI_ACTIVE" in names
                else "")]
    head = f"{'kernel':58s} {'wgs':>7s} {'wg':>5s} {'n':>4s} {'us':>9s} " + " ".join(f"{c:>20s}" for c in cols)
    extra = []
    if "GRBM_GUI_ACTIVE" in names:
        extra.append("clock_MHz")
    if {"SQ_WAVES", "SQ_INSTS_VALU"} <= names:
        extra.append("valu_per_wave")
    if {"GRBM_GUI_ACTIVE", "SQ_INSTS_VALU"} <= names:
        extra.append("valu_busy")
    if {"GRBM_GUI_ACTIVE", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES"} <= names:
        extra += ["mfma_busy", "valu_per_mfma"]
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in names:
            extra.append("coexec")
    if hbm_bytes and "GRBM_GUI_ACTIVE" in names:
        extra += ["hbm_GBps", "hbm_B_per_clk"]
    lines.append(head + "".join(f" {e:>14s}" for e in extra))
    for key in sorted(vals, key=lambda k: -st.mean(durs[k].values()) if durs[k] else 0):
        d = list(durs[key].values())
        us = st.mean(d) if d else float("nan")
        means = {c: st.mean(vals[key][c]) if vals[key][c] else float("nan") for c in cols}
        line = f"{key[0][:58]:58s} {key[1]:7d} {key[2]:5d} {len(d):4d} {us:9.2f} " + \
            " ".join(f"{means[c]:20.1f}" for c in cols)
        if "clock_MHz" in extra:
            line += f" {means['GRBM_GUI_ACTIVE'] / XCDS / us:14.1f}"
        if "valu_per_wave" in extra:
            line += f" {means['SQ_INSTS_VALU'] / max(means['SQ_WAVES'], 1.0):14.1f}"
        if "valu_busy" in extra:
            line += f" {means['SQ_INSTS_VALU'] * 4 / (SIMDS * means['GRBM_GUI_ACTIVE'] / XCDS):14.3f}"
        if "mfma_busy" in extra:
            mb = means["SQ_VALU_MFMA_BUSY_CYCLES"]
            mi = means["SQ_INSTS_MFMA"]
            line += f" {mb / (SIMDS * means['GRBM_GUI_ACTIVE'] / XCDS):14.3f}"
            line += f" {(means['SQ_INSTS_VALU'] - mi) / mi:14.2f}" if mi > 0 else f" {'-':>14s}"
            if "coexec" in extra:
                line += f" {means['SQ_VALU_MFMA_COEXEC_CYCLES'] / mb:14.3f}" if mb > 0 else f" {'-':>14s}"
        if "hbm_GBps" in extra:
            b = hbm_bytes.get(key)
            if b is None:
                line += f" {'-':>14s} {'-':>14s}"
            else:
                line += f" {b / us / 1e3:14.1f} {b / (means['GRBM_GUI_ACTIVE'] / XCDS):14.1f}"
        lines.append(line)
    return "\n".join(lines)


def traffic_summary(fetch_dir: str, write_dir: str):
    fetch, nf = _counter_means(fetch_dir, "FETCH_SIZE")
    write, nw = _counter_means(write_dir, "WRITE_SIZE")
    # calibration: the torch.neg dispatches (exactly 256 MiB read and written)
    def calib(d):
        cands = [(k, v) for k, v in d.items() if "neg" in k[0].lower()]
        if not cands:
            raise SystemExit("no torch.neg calibration dispatch in the counter output "
                             "(run bench.py with --calib-copy)")
        return max(cands, key=lambda kv: kv[1])
    cf, cw = calib(fetch), calib(write)
    f_scale = CALIB_BYTES / cf[1]
    w_scale = CALIB_BYTES / cw[1]
    out = {"fetch_scale": f_scale, "write_scale": w_scale,
           "fetch_calibration_kernel": cf[0][0] if cf else None,
           "write_calibration_kernel": cw[0][0] if cw else None, "kernels": {}}
    lines = [f"calibration (torch.neg over 256 MiB: {cf[0][0][:50]}): FETCH_SIZE x {f_scale:.4f}, "
             f"WRITE_SIZE x {w_scale:.4f}",
             f"{'kernel':58s} {'workgroups':>10s} {'wg':>4s} {'n':>4s} {'fetch_MB':>10s} {'write_MB':>10s}"]
    for k in sorted(set(fetch) | set(write), key=lambda k: -fetch.get(k, 0)):
        fb = fetch.get(k, 0.0) * f_scale
        wb = write.get(k, 0.0) * w_scale
        lines.append(f"{k[0][:58]:58s} {k[1]:10d} {k[2]:4d} {nf.get(k, 0):4d} {fb / 1e6:10.3f} {wb / 1e6:10.3f}")
        out["kernels"][f"{k[0]}|{k[1]}x{k[2]}"] = {"fetch_bytes": fb, "write_bytes": wb}
    return "\n".join(lines), out


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STEP_ARGS = ["--no-configs", "--no-cpu", "--no-q8-step", "--no-graph", "--steps", "100", "--warmup", "15"]
CALL_ARGS = ["--no-cpu", "--no-graph", "--no-warm", "--steps", "20", "--warmup", "5", "--reps", "60"]
PMC_ARGS = ["--no-cpu", "--no-graph", "--no-warm", "--calib-copy", "--steps", "3", "--warmup", "2", "--reps", "5",
            "--only", "c0,c1,c2,c3,c4,k"]
SQ_COUNTERS = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CYCLES", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"]
# the prefill GEMM rows only (the headline step runs a few steps first)
GEMM_ARGS = ["--no-cpu", "--no-graph", "--no-q8-step", "--steps", "3", "--warmup", "2", "--reps", "3", "--settle-ms",
             "20", "--only", "g "]
MFMA_COUNTERS = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES",
                 "SQ_INSTS_SALU", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"]
# the headline step's calls: bench.py label -> the kernel launch shape that runs it
STEP_CALLS = {"gate|up 2x17408x5120 silu": "qgk::qgemv_kernel<2, 1, 1, 1, true, 1, false>|1088x256",
              "down 5120x17408": "qgk::qgemv_persist<2, 1, 0, true, false, false, true>|256x1024",
              "lm_head 248320x5120": "qgk::qgemv_kernel<2, 1, 0, 1, true, 1, false>|7760x256"}


def _run_pass(name: str, prof_args: list, bench_args: list, out: str, limit: int):
    """One rocprofv3 pass over bench.py; returns (command string, bench JSON line or None)."""
    import subprocess
    d = os.path.join(out, name)
    cmd = ["timeout", "-s", "KILL", str(limit), "rocprofv3", *prof_args, "-f", "csv", "-d", d, "-o", "run", "--",
           sys.executable, os.path.join(ROOT, "bench.py"), *bench_args]
    shown = " ".join(["rocprofv3", *prof_args, "-f", "csv", "-d", f"<out>/{name}", "-o", "run", "--", "python3",
                      "bench.py", *bench_args])
    print(f"[prof] pass {name}: {shown}", file=sys.stderr, flush=True)
    with open(os.path.join(out, name + ".log"), "w") as log:
        r = subprocess.run(cmd, cwd="/tmp", stdout=subprocess.PIPE, stderr=log, text=True,
                           env={**os.environ, "TMPDIR": "/tmp"})
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith('{"metric"')]
    # rocprofv3 can exit 139 on its own after the program finished (its JSON line printed)
    if r.returncode != 0 and not (r.returncode in (139, -11) and lines):
        raise SystemExit(f"pass {name} failed with status {r.returncode} (see {name}.log)")
    return shown, (json.loads(lines[-1]) if lines else None)


def collect(out: str, only=None):
    """Run the profiler passes (all, or those named in `only`) and write their summaries."""
    out = os.path.abspath(out)   # the passes run from /tmp
    os.makedirs(out, exist_ok=True)
    summaries = {}
    want = lambda name: only is None or name in only  # noqa: E731
    if want("trace_step"):
        cmd, res = _run_pass("trace_step", ["--kernel-trace", "--stats"], STEP_ARGS, out, 600)
        roof = res["roofline"] if res else {}
        k = roof.get("launches")
        summaries["trace_step"] = (
            f"command: {cmd}\n"
            f"summaries: python -m block_dequant_gemv_amd.prof trace <out>/trace_step --tail {k}\n"
            f"           python -m block_dequant_gemv_amd.prof trace <out>/trace_step --skip 15\n"
            f"the same run's bench.py: step {res.get('ms_per_step') if res else None} ms, "
            f"{res.get('value') if res else None} GB/s (plain launches); roofline {roof.get('call')}: "
            f"{roof.get('avg_launch_us')} us per launch over {k} launches back to back between two events, "
            f"{roof.get('achieved')} GB/s = {roof.get('frac')} of 8 TB/s\n\n"
            f"the back-to-back launches the roofline is taken from (the last {k} of every launch shape):\n"
            + trace_summary(os.path.join(out, "trace_step"), 0, k or 0, stats_csv=False)
            + "\n\nevery launch after the warm-up (timed steps, the bound-event pass and the back-to-back batches):\n"
            + trace_summary(os.path.join(out, "trace_step"), 15))
    if want("trace_calls"):
        cmd, _ = _run_pass("trace_calls", ["--kernel-trace", "--stats"], CALL_ARGS, out, 900)
        summaries["trace_calls"] = (f"command: {cmd}\nsummary: python -m block_dequant_gemv_amd.prof trace "
                                    f"<out>/trace_calls --skip 3\n\n" + trace_summary(os.path.join(out, "trace_calls"), 3))
    if want("traffic"):
        cmd_f, _ = _run_pass("fetch", ["--pmc", "FETCH_SIZE"], PMC_ARGS, out, 600)
        cmd_w, _ = _run_pass("write", ["--pmc", "WRITE_SIZE"], PMC_ARGS, out, 600)
        text, data = traffic_summary(os.path.join(out, "fetch"), os.path.join(out, "write"))
        data["kernel_source_hash"] = kernel_source_hash()
        data["calls"] = {}
        for label, key in STEP_CALLS.items():
            k = data["kernels"].get(key)
            if k:
                data["calls"][label] = {"kernel": key, "fetch_bytes": k["fetch_bytes"], "write_bytes": k["write_bytes"],
                                        "bytes_per_launch": k["fetch_bytes"] + k["write_bytes"]}
        with open(os.path.join(out, "traffic.json"), "w") as f:
            json.dump(data, f, indent=1)
        summaries["traffic"] = (f"commands: {cmd_f}\n          {cmd_w}\nsummary: python -m block_dequant_gemv_amd.prof "
                                f"traffic <out>/fetch <out>/write\n\n" + text)
    if want("sq"):
        cmd, _ = _run_pass("sq", ["--pmc", *SQ_COUNTERS, "--kernel-trace"], PMC_ARGS, out, 600)
        hbm = None
        if os.path.exists(os.path.join(out, "traffic.json")):
            with open(os.path.join(out, "traffic.json")) as f:
                hbm = shape_bytes(json.load(f))
        summaries["sq"] = (f"command: {cmd}\nsummary: python -m block_dequant_gemv_amd.prof counters <out>/sq"
                           + (" <out>/traffic.json" if hbm else "") + "\n\n"
                           + counter_summary(os.path.join(out, "sq"), hbm))
    if want("trace_gemm"):
        cmd, _ = _run_pass("trace_gemm", ["--kernel-trace", "--stats"], GEMM_ARGS, out, 600)
        summaries["trace_gemm"] = (f"command: {cmd}\nsummary: python -m block_dequant_gemv_amd.prof trace "
                                   f"<out>/trace_gemm --skip 3\n\n" + trace_summary(os.path.join(out, "trace_gemm"), 3))
    if want("gemm_sq"):
        cmd, _ = _run_pass("gemm_sq", ["--pmc", *MFMA_COUNTERS, "--kernel-trace"], GEMM_ARGS, out, 600)
        summaries["gemm_sq"] = (f"command: {cmd}\nsummary: python -m block_dequant_gemv_amd.prof counters "
                                f"<out>/gemm_sq\n\n" + counter_summary(os.path.join(out, "gemm_sq")))
    for name, text in summaries.items():
        with open(os.path.join(out, name + ".txt"), "w") as f:
            f.write(text + "\n")
    print(f"[prof] summaries in {out}", file=sys.stderr)


def main(argv):
    if len(argv) >= 2 and argv[0] == "trace":
        skip = int(argv[argv.index("--skip") + 1]) if "--skip" in argv else 0
        tail = int(argv[argv.index("--tail") + 1]) if "--tail" in argv else 0
        print(trace_summary(argv[1], skip, tail))
    elif len(argv) >= 2 and argv[0] == "counters":
        hbm = None
        if len(argv) >= 3:
            with open(argv[2]) as f:
                hbm = shape_bytes(json.load(f))
        print(counter_summary(argv[1], hbm))
    elif len(argv) >= 2 and argv[0] == "collect":
        collect(argv[1], argv[argv.index("--only") + 1].split(",") if "--only" in argv else None)
    elif len(argv) >= 3 and argv[0] == "traffic":
        text, data = traffic_summary(argv[1], argv[2])
        print(text)
        data["kernel_source_hash"] = kernel_source_hash()
        data["calls"] = {}
        for i, a in enumerate(argv):
            if a == "--call":
                label, key = argv[i + 1].split("=", 1)
                k = data["kernels"][key]
                data["calls"][label] = {"kernel": key, "fetch_bytes": k["fetch_bytes"], "write_bytes": k["write_bytes"],
                                        "bytes_per_launch": k["fetch_bytes"] + k["write_bytes"]}
        if "--json" in argv:
            with open(argv[argv.index("--json") + 1], "w") as f:
                json.dump(data, f, indent=1)
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
