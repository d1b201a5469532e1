"""Benchmark of the fused exact-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]

One step is one fused forward (load Q tile, stream K/V tiles, scores on
MFMA, online softmax, P V on MFMA, O/l and LSE) over one batch of seeded
synthetic inputs already resident in device memory.  Prints ONE JSON line:
whole-job TFLOP/s (4*B*H*N^2*d per step / time), the roofline of the fused
kernel (MFMA-bound; achieved = algorithmic FLOPs per launch / mean launch
time from HIP events on the launch stream), the naive three-kernel path
timed on the same inputs as a contrast, and the fp64 CPU oracle timed on a
bounded sample of the same workload on this host's cores.
"""

import argparse
import hashlib
import json
import math
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd attention TFLOP/s (4BHN²d/t) + % bf16 MFMA peak, N=4096 d=128"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16/fp16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2      # MI355X dense fp8 MFMA: twice the bf16 rate
PEAK_HBM_GBS = 8000.0
FUSED_KERNEL_SOURCES = ["io_aware_softmax_04_amd/csrc/fa_fwd_gfx950.hip",
                        "io_aware_softmax_04_amd/csrc/fa_device.h",
                        "io_aware_softmax_04_amd/csrc/fa_sched.h"]
TRAFFIC_FILE = "profiles/traffic_fused_fwd_{tag}.md"
FUSED_KERNEL_NAME = "fa_fwd_16_kernel"
COPY_KERNEL_NAME = "__amd_rocclr_copyBuffer"
NAIVE_KERNEL_NAMES = ["naive_scores_16", "naive_softmax_16", "naive_pv_16"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # the GPU's clock and power state settle within a few hundred
    # milliseconds of sustained load (the first ~30 ms run about 12% slower),
    # so the default warm-up covers about 0.6 s before the timed steps
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=2000)
    p.add_argument("--workload", type=int, default=3)
    p.add_argument("--no-naive", action="store_true", help="skip the naive contrast")
    p.add_argument("--no-splitkv", action="store_true", help="skip the split-KV contrast")
    p.add_argument("--no-decode", action="store_true", help="skip the decode measurement")
    p.add_argument("--no-softmax", action="store_true", help="skip the row-softmax measurement")
    p.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    p.add_argument("--no-fp8", action="store_true", help="skip the FP8 forward measurement")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the sustained-MFMA ceiling measurement")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="also run a device copy of this many MiB (counter calibration)")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                        "`bench.py --calibrate-copy-mib M` into the traffic summary under "
                        "profiles/ and exit (no GPU needed)")
    p.add_argument("--trace-from", metavar="TRACE_DIR",
                   help="summarise a `rocprofv3 --kernel-trace --stats` run of bench.py "
                        "into the kernel-trace summary under profiles/ and exit")
    p.add_argument("--trace-cmd", default="",
                   help="the bench.py arguments of that run (recorded in the summary)")
    p.add_argument("--sq-from", nargs="+", metavar="PMC_DIR",
                   help="summarise one or two `rocprofv3 --pmc` passes of bench.py (the "
                        "counter sets SQ_PASSES a and b) into the shader-counter summary of "
                        "--sq-kernel under profiles/ (effective clock, MFMA busy, waits) and exit")
    p.add_argument("--sq-kernel", default="fused", choices=sorted(SQ_KERNELS),
                   help="kernel the counter summary covers")
    p.add_argument("--copy-mib", type=int, default=1024,
                   help="size of the calibration copy in those runs")
    p.add_argument("--sweep-splits", action="store_true",
                   help="time the split-KV forward at every split count of the sweep lists "
                        "and write the tables to " + SWEEP_FILE + ", then exit")
    return p.parse_args()


def sources_hash():
    h = hashlib.sha256()
    for rel in FUSED_KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def workload_tag(spec):
    return f"{spec['dtype']}_B{spec['B']}H{spec['H']}N{spec['N']}d{spec['d']}"


def bytes_models(spec, br=128):
    """Algorithmic byte counts per forward (whole job)."""
    e = 4 if spec["dtype"] == "fp32" else 2
    B, H, N, d = spec["B"], spec["H"], spec["N"], spec["d"]
    heads = B * H
    return {
        "compulsory": heads * (e * 4 * N * d + 4 * N),
        "tiled_io_model": heads * (e * (2 * N * d + 2 * N * d * math.ceil(N / br)) + 4 * N),
        "naive_model": heads * e * (4 * N * d + 4 * N * N),
    }


def fused_grid_items(spec):
    """Work-items of the fused kernel's launch at the workload (its grid as
    the profiler reports it), which tells its dispatches apart from launches
    of the same kernel on other shapes in the same run (the split-KV
    contrast's head share).  16-bit inputs: workgroups of 8 waves (256 query
    rows) at d = 128 when there are at least as many of them as CUs (256),
    else of 4 waves (128 rows)."""
    heads = spec["B"] * spec["H"]
    waves = 8 if spec["d"] == 128 and heads * math.ceil(spec["N"] / 256) >= 256 else 4
    return heads * math.ceil(spec["N"] / (32 * waves)) * 64 * waves


# fa_fwd_16_kernel<T, D, BC, PARTIAL, waves>: the fused forward proper has
# PARTIAL = false (the split-KV partial pass is true)
_FUSED_FULL = re.compile(FUSED_KERNEL_NAME + r"<[^<>]*?, \d+, \d+, false(?:, \d+)?>")


def _is_fused(row, spec, grid_key="Grid_Size"):
    return (_FUSED_FULL.search(row["Kernel_Name"]) is not None
            and int(row[grid_key]) == fused_grid_items(spec))


def _counter_rows(directory, counter):
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    rows = []
    for f in files:
        with open(f, encoding="utf-8") as fh:
            rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
    return rows


def summarise_traffic(fetch_dir, write_dir, copy_mib, index, spec):
    """HBM-side bytes of the fused kernel from the FETCH_SIZE and WRITE_SIZE
    counters (KiB per dispatch), each scaled so that a device copy of
    ``copy_mib`` MiB reads and writes exactly that many bytes."""
    copy_bytes = copy_mib * (1 << 20)
    out = {}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(directory, counter)
        fused = [float(r["Counter_Value"]) for r in rows if _is_fused(r, spec)]
        copy = [float(r["Counter_Value"]) for r in rows if COPY_KERNEL_NAME in r["Kernel_Name"]]
        if not fused or not copy:
            raise SystemExit(f"{counter}: fused or calibration-copy dispatches missing")
        # the runtime may run the one calibration copy as several dispatches:
        # their counts add up (other copies in the run are a few KiB)
        factor = copy_bytes / (sum(copy) * 1024)
        kib = sum(fused) / len(fused)
        out[counter] = dict(kib=kib, factor=factor, bytes=kib * 1024 * factor,
                            dispatches=len(fused), copy_kib=sum(copy),
                            copy_dispatches=len(copy))
    total = out["FETCH_SIZE"]["bytes"] + out["WRITE_SIZE"]["bytes"]
    # the naive contrast's three kernels, if the runs included them
    naive = {}
    for counter, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for r in _counter_rows(directory, counter):
            for kname in NAIVE_KERNEL_NAMES:
                if kname in r["Kernel_Name"]:
                    naive.setdefault(kname, {}).setdefault(counter, []).append(
                        float(r["Counter_Value"]) * 1024 * out[counter]["factor"])
    models = bytes_models(spec)
    tag = workload_tag(spec)
    lines = [
        f"# HBM traffic of the fused forward, {spec['name']}",
        "",
        "Commands (one MI355X, from the repository root; one counter per run):",
        "",
        "```",
        f"rocprofv3 --pmc FETCH_SIZE -d {fetch_dir} -o run --output-format csv -- "
        f"python bench.py --workload {index} {TRAFFIC_BENCH_ARGS} --calibrate-copy-mib {copy_mib}",
        f"rocprofv3 --pmc WRITE_SIZE -d {write_dir} -o run --output-format csv -- "
        f"python bench.py --workload {index} {TRAFFIC_BENCH_ARGS} --calibrate-copy-mib {copy_mib}",
        f"python bench.py --workload {index} --traffic-from "
        f"{fetch_dir} {write_dir} --copy-mib {copy_mib}",
        "```",
        "",
        f"Calibration: a device copy of {copy_mib} MiB ({COPY_KERNEL_NAME}, "
        f"{out['FETCH_SIZE']['copy_dispatches']} and {out['WRITE_SIZE']['copy_dispatches']} "
        f"dispatches of that kernel in the two runs, counts summed) reads "
        f"{out['FETCH_SIZE']['copy_kib']:.1f} KiB on FETCH_SIZE and writes "
        f"{out['WRITE_SIZE']['copy_kib']:.1f} KiB on WRITE_SIZE, so the counters are "
        f"scaled by {out['FETCH_SIZE']['factor']:.4f} (fetch) and "
        f"{out['WRITE_SIZE']['factor']:.4f} (write).",
        "",
        "| counter | KiB / dispatch (raw) | dispatches | scale | bytes / launch |",
        "|---|---|---|---|---|",
    ]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        r = out[c]
        lines.append(f"| {c} | {r['kib']:.2f} | {r['dispatches']} | {r['factor']:.4f} | "
                     f"{r['bytes']:.0f} |")
    lines += [
        "",
        f"Total {total:.0f} bytes per launch: {total / models['compulsory']:.3f} x the "
        f"compulsory bytes ({models['compulsory']}), {total / models['tiled_io_model']:.4f} x "
        f"the tiled-IO model at Br=128 ({models['tiled_io_model']}), "
        f"{total / models['naive_model']:.4f} x the naive model ({models['naive_model']}).",
        "",
    ]
    if naive:
        lines += [
            "Naive three-kernel contrast in the same runs (bytes per launch, scaled as above):",
            "",
            "| kernel | read | written | total |",
            "|---|---|---|---|",
        ]
        ntotal = 0.0
        for kname in NAIVE_KERNEL_NAMES:
            if kname not in naive:
                continue
            rd = sum(naive[kname]["FETCH_SIZE"]) / len(naive[kname]["FETCH_SIZE"])
            wr = sum(naive[kname]["WRITE_SIZE"]) / len(naive[kname]["WRITE_SIZE"])
            ntotal += rd + wr
            lines.append(f"| {kname} | {rd:.0f} | {wr:.0f} | {rd + wr:.0f} |")
        lines += [
            "",
            f"Naive total {ntotal:.0f} bytes = {ntotal / models['naive_model']:.3f} x the "
            f"element-count model e*B*H*(4Nd + 4N^2) = {models['naive_model']}; the fused "
            f"kernel moves {total / ntotal:.4f} x the naive path's bytes.",
            "",
        ]
    lines += [
        "Machine-readable (bench.py reads these two lines; the hash covers the fused "
        "kernel's sources, so the figure is dropped once the kernel changes):",
        "",
        f"bytes_per_launch: {total:.0f}",
        f"kernel_sources_sha256_16: {sources_hash()}",
        "",
    ]
    path = os.path.join(ROOT, TRAFFIC_FILE.format(tag=tag))
    with open(path, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines))
    print(path)


def summarise_trace(trace_dir, index, spec, bench_args, out_dir=None):
    """Per-kernel durations from rocprofv3's kernel_trace.csv, one row per
    kernel and launch grid, with the fused kernel's rate at the algorithmic
    FLOP count for the workload's grid.  When the profiled run's stdout was
    kept beside the trace, its bench line's HIP-event launch average is quoted
    next to the trace's average.  Writes profiles/kernel_trace_<tag>.md (or
    into out_dir) and returns its path."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    groups = {}
    with open(files[0], encoding="utf-8") as fh:
        for r in csv.DictReader(fh):
            key = (r["Kernel_Name"], int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"])
                   * int(r["Grid_Size_Z"]))
            groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    flops = 4.0 * spec["B"] * spec["H"] * spec["N"] ** 2 * spec["d"]
    tag = workload_tag(spec)
    # the profiled run's own JSON line, when its stdout was kept beside the trace
    bench_line = None
    out_path = os.path.join(trace_dir, BENCH_STDOUT)
    if os.path.exists(out_path):
        with open(out_path, encoding="utf-8") as fh:
            rows = [ln for ln in fh if ln.startswith("{")]
        if rows:
            bench_line = json.loads(rows[-1])
    redirect = f" > {out_path}" if bench_line is not None else ""
    lines = [
        f"# Kernel trace, {spec['name']}",
        "",
        "Command (one MI355X, from the repository root):",
        "",
        "```",
        f"rocprofv3 --kernel-trace --stats -d {trace_dir} -o run --output-format csv -- "
        f"python bench.py {bench_args}{redirect}",
        f"python bench.py --workload {index} --trace-from {trace_dir} --trace-cmd='{bench_args}'",
        "```",
        "",
        f"One row per kernel and launch grid (work-items); the fused forward at this "
        f"workload launches {fused_grid_items(spec)} work-items, other grids of the same "
        f"kernel belong to the split-KV contrast's head share.",
        "",
        "| kernel | grid | calls | average (ns) | min (ns) | max (ns) | TFLOP/s at 4BHN^2d |",
        "|---|---|---|---|---|---|---|",
    ]
    fused_avg_ns = None
    for (name, grid), ns in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        short = name.replace("(anonymous namespace)::", "").split("(")[0]
        short = short.replace("void ", "").replace("iofa::", "")
        if short.startswith("at::native"):
            short = short.split("<")[0]
        rate = ""
        if _is_fused({"Kernel_Name": name, "Grid_Size": grid}, spec):
            rate = f"{flops / (sum(ns) / len(ns) * 1e-9) / 1e12:.1f}"
            fused_avg_ns = sum(ns) / len(ns)
        lines.append(f"| {short} | {grid} | {len(ns)} | {sum(ns) / len(ns):.0f} | {min(ns)} | "
                     f"{max(ns)} | {rate} |")
    if bench_line is not None and fused_avg_ns is not None:
        ev_ms = bench_line["fused_launch_ms"]
        lines += [
            "",
            "The same run's bench line timed the fused launches with HIP events on the launch "
            f"stream: mean {ev_ms:.5f} ms (median {bench_line['fused_launch_ms_median']:.5f}), "
            f"roofline.achieved {bench_line['roofline']['achieved']} TFLOP/s; the kernel "
            f"trace's average of all the fused dispatches above is {fused_avg_ns * 1e-6:.5f} ms "
            f"(trace / events = {fused_avg_ns * 1e-6 / ev_ms:.3f}).",
        ]
    lines += ["", f"kernel_sources_sha256_16: {sources_hash()}", ""]
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"kernel_trace_{tag}.md")
    with open(path, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines))
    print(path)
    return path


# file name of a profiled run's stdout kept beside its kernel trace
BENCH_STDOUT = "bench_stdout.txt"

# the traffic passes run the fused and the naive paths only, a few launches each
TRAFFIC_BENCH_ARGS = ("--steps 3 --warmup 1 --no-splitkv --no-decode --no-softmax --no-backward "
                      "--no-fp8 --no-ceiling --no-cpu-baseline")
# Shader counters, in rocprofv3 --pmc passes of at most 8 SQ counters each
# (a and b for every kernel; c, the LDS pass, optional)
SQ_PASSES = {
    "a": ["SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
          "SQ_INSTS_LDS", "SQ_INSTS_VALU_TRANS_F32", "SQ_WAVES", "SQ_WAVE_CYCLES"],
    "b": ["SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_LDS",
          "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
          "SQ_INSTS_SALU"],
    "c": ["SQ_BUSY_CYCLES", "SQ_INSTS_LDS", "SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_LDS_IDX_ACTIVE",
          "SQ_LDS_BANK_CONFLICT", "SQ_LDS_ADDR_CONFLICT", "SQ_LDS_CMD_FIFO_FULL",
          "SQ_LDS_DATA_FIFO_FULL"],
}
COMPUTE_UNITS = 256
SHADER_ENGINES = 32          # 8 XCDs x 4 shader engines
SIMDS = 1024                 # 256 CUs x 4
# Kernels the counter summary covers: (name filter, FLOPs per MFMA instruction,
# bench.py arguments of the counter passes, file tag, rocprofv3 kernel regex)
_SQ_COMMON = ("--warmup 100 --no-naive --no-splitkv --no-decode --no-softmax --no-ceiling "
              "--no-cpu-baseline")
SQ_KERNELS = {
    "fused": ("fused", 32768.0, f"--steps 20 {_SQ_COMMON} --no-backward --no-fp8", "fused_fwd",
              "fa_fwd_16_kernel"),
    "bwd_dq": ("bwd_dq_kernel", 32768.0, f"--steps 20 {_SQ_COMMON} --no-fp8", "bwd_dq",
               "bwd_dq_kernel"),
    "bwd_dkdv": ("bwd_dkdv_kernel", 32768.0, f"--steps 20 {_SQ_COMMON} --no-fp8", "bwd_dkdv",
                 "bwd_dkdv_kernel"),
    "fp8": ("fa_fwd_fp8_kernel", 131072.0, f"--steps 20 {_SQ_COMMON} --no-backward", "fp8_fwd",
            "fa_fwd_fp8_kernel"),
}


def _sq_match(row, spec, which):
    name = SQ_KERNELS[which][0]
    if name == "fused":
        return _is_fused(row, spec)
    return name in row["Kernel_Name"]


def summarise_sq(pmc_dirs, index, spec, which="fused", out_dir=None):
    """Shader counters of one kernel from one or more rocprofv3 --pmc passes.

    SQ_BUSY_CYCLES counts, per shader engine, the cycles any wave is
    resident; summed over the 32 engines and divided by 32 it is the
    kernel's length in shader cycles, so dividing by the dispatch's duration
    gives the clock it ran at.  SQ_VALU_MFMA_BUSY_CYCLES summed over the
    SIMDs, over SIMDs x kernel cycles, is the fraction of time the matrix
    cores were busy; SQ_VALU_MFMA_COEXEC_CYCLES likewise the fraction in
    which a vector instruction issued while they were busy.  SQ_WAVE_CYCLES,
    SQ_WAIT_ANY and SQ_WAIT_INST_LDS are wave-cycles in units of 4 cycles:
    their ratios are the fraction of a wave's lifetime spent waiting, and
    waiting to issue an LDS instruction.  From the optional third pass:
    SQ_INSTS_LDS_LOAD_BANDWIDTH counts 64-byte units read from LDS, and
    SQ_LDS_IDX_ACTIVE the cycles the CUs' LDS spent on indexed accesses
    (summed over CUs), so their ratio is the bytes the LDS returned per
    active cycle and the latter over CUs x kernel cycles its busy fraction."""
    import csv
    import glob
    per = {}
    for d in pmc_dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        for f in files:
            with open(f, encoding="utf-8") as fh:
                rows = [r for r in csv.DictReader(fh) if _sq_match(r, spec, which)]
            # dispatches of one pass, in order; passes are matched by position
            ids = sorted({int(r["Dispatch_Id"]) for r in rows})
            pos = {i: n for n, i in enumerate(ids)}
            for r in rows:
                e = per.setdefault(pos[int(r["Dispatch_Id"])], {})
                e[r["Counter_Name"]] = float(r["Counter_Value"])
                e.setdefault("ns", []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if not per:
        raise SystemExit(f"no {which} dispatches in the counter runs")
    # each counter is averaged over the dispatches that carry it (the passes
    # need not hold the same number of dispatches)
    keys = sorted(per)
    names = set().union(*(set(v) for v in per.values())) - {"ns"}
    avg = {}
    for c in names:
        vals = [per[k][c] for k in keys if c in per[k]]
        avg[c] = sum(vals) / len(vals)
    avg["ns"] = sum(sum(per[k]["ns"]) / len(per[k]["ns"]) for k in keys) / len(keys)
    cycles = avg["SQ_BUSY_CYCLES"] / SHADER_ENGINES
    mhz = cycles / (avg["ns"] * 1e-3)
    _, flops_per_mfma, bench_args, tag, regex = SQ_KERNELS[which]
    lines = [
        f"# Shader counters of {which} ({SQ_KERNELS[which][0]}), {spec['name']}",
        "",
        "Commands (one MI355X, from the repository root; one pass per counter set):",
        "",
        "```",
    ]
    for name, d in zip(("a", "b", "c"), pmc_dirs):
        lines.append(f"rocprofv3 --pmc {' '.join(SQ_PASSES[name])} --kernel-include-regex "
                     f"'{regex}' -d {d} -o run --output-format csv "
                     f"-- python bench.py --workload {index} {bench_args}")
    lines += [f"python bench.py --workload {index} --sq-kernel {which} --sq-from "
              f"{' '.join(pmc_dirs)}", "```", "",
              f"Averages over {len(keys)} dispatches:", "", "| quantity | value |", "|---|---|"]
    mfma = avg.get("SQ_INSTS_MFMA")
    tflops = mfma * flops_per_mfma / (avg["ns"] * 1e-9) / 1e12 if mfma else None
    lines.append(f"| dispatch duration | {avg['ns'] / 1e3:.1f} us |")
    if tflops:
        lines.append(f"| executed MFMA rate (SQ_INSTS_MFMA x {flops_per_mfma:.0f} FLOP) | "
                     f"{tflops:.1f} TFLOP/s |")
    lines += [f"| SQ_BUSY_CYCLES / 32 engines | {cycles:.0f} shader cycles |",
              f"| effective shader clock | {mhz:.0f} MHz (nominal peak clock 2400 MHz) |"]
    if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * cycles)
        lines.append(f"| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / SIMDs / cycles) | {busy:.3f} |")
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
        lines.append(f"| vector issue while MFMA busy (COEXEC / SIMDs / cycles) | "
                     f"{avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / (SIMDS * cycles):.3f} |")
    if "SQ_ACTIVE_INST_VALU" in avg:
        lines.append(f"| vector instructions active (4 x ACTIVE_INST_VALU / SIMDs / cycles) | "
                     f"{4 * avg['SQ_ACTIVE_INST_VALU'] / (SIMDS * cycles):.3f} |")
    if "SQ_ACTIVE_INST_LDS" in avg:
        lines.append(f"| LDS instructions active (4 x ACTIVE_INST_LDS / SIMDs / cycles) | "
                     f"{4 * avg['SQ_ACTIVE_INST_LDS'] / (SIMDS * cycles):.3f} |")
    if "SQ_WAIT_ANY" in avg:
        lines.append(f"| wave lifetime spent waiting (WAIT_ANY / WAVE_CYCLES) | "
                     f"{avg['SQ_WAIT_ANY'] / avg['SQ_WAVE_CYCLES']:.3f} |")
        lines.append(f"| wave lifetime waiting to issue LDS (WAIT_INST_LDS / WAVE_CYCLES) | "
                     f"{avg['SQ_WAIT_INST_LDS'] / avg['SQ_WAVE_CYCLES']:.3f} |")
    if "SQ_WAVES" in avg:
        waves = avg["SQ_WAVES"]
        lines.append(f"| waves | {waves:.0f} |")
        lines.append(f"| per wave: MFMA / VALU (incl. MFMA) / transcendental / LDS instructions | "
                     f"{mfma / waves:.0f} / {avg['SQ_INSTS_VALU'] / waves:.0f} / "
                     f"{avg['SQ_INSTS_VALU_TRANS_F32'] / waves:.0f} / "
                     f"{avg['SQ_INSTS_LDS'] / waves:.0f} |")
        lines.append(f"| non-MFMA VALU + LDS instructions per MFMA | "
                     f"{(avg['SQ_INSTS_VALU'] - mfma + avg['SQ_INSTS_LDS']) / mfma:.2f} |")
        if "SQ_INSTS_SALU" in avg:
            lines.append(f"| scalar instructions per wave | {avg['SQ_INSTS_SALU'] / waves:.0f} |")
    if "SQ_LDS_IDX_ACTIVE" in avg:
        lds_bytes = 64.0 * avg["SQ_INSTS_LDS_LOAD_BANDWIDTH"]
        active = avg["SQ_LDS_IDX_ACTIVE"]
        lines += [f"| LDS bytes read per dispatch (64 x SQ_INSTS_LDS_LOAD_BANDWIDTH) | "
                  f"{lds_bytes:.4g} |",
                  f"| LDS bytes per active cycle (bytes / SQ_LDS_IDX_ACTIVE) | "
                  f"{lds_bytes / active:.0f} |",
                  f"| LDS busy (SQ_LDS_IDX_ACTIVE / CUs / cycles) | "
                  f"{active / (COMPUTE_UNITS * cycles):.3f} |",
                  f"| LDS bank / address conflict cycles per active cycle | "
                  f"{avg['SQ_LDS_BANK_CONFLICT'] / active:.3f} / "
                  f"{avg['SQ_LDS_ADDR_CONFLICT'] / active:.3f} |",
                  f"| LDS command / data FIFO full cycles per active cycle | "
                  f"{avg['SQ_LDS_CMD_FIFO_FULL'] / active:.4f} / "
                  f"{avg['SQ_LDS_DATA_FIFO_FULL'] / active:.4f} |"]
    lines += ["", f"kernel_sources_sha256_16: {sources_hash()}", ""]
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"),
                        f"sq_counters_{tag}_{workload_tag(spec)}.md")
    with open(path, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines))
    print(path)
    return path


def read_traffic(spec):
    """bytes_per_launch from the committed traffic summary, or None when it is
    missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_FILE.format(tag=workload_tag(spec)))
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path, encoding="utf-8") as fh:
        for ln in fh:
            if ":" in ln and not ln.startswith(("|", "#", "`")):
                key, _, val = ln.partition(":")
                fields[key.strip()] = val.strip()
    if fields.get("kernel_sources_sha256_16") != sources_hash():
        return None
    return int(fields["bytes_per_launch"])


def time_launches(fn, steps, warmup, torch, warm_seconds=0.0):
    """Run ``fn`` warmup times (then keep running it until ``warm_seconds``
    have passed, so the GPU's clock has settled under load), then time
    ``steps`` back-to-back calls between two synchronisations (wall clock,
    nothing else queued between the launches), then ``steps`` more calls
    with HIP events recorded on the launch stream around each one.  Returns
    (wall ms per step, mean launch ms from the events, the events' median
    and minimum in ms)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + warm_seconds
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    times = sorted(a.elapsed_time(b) for a, b in evs)
    ev = sum(times) / steps
    return wall, ev, times[steps // 2], times[0]


def time_graph(fn, torch, reps=20, replays=10, warm_seconds=0.3):
    """Mean duration of one call of ``fn`` when ``reps`` calls are captured
    in one graph and the graph is replayed ``replays`` times between two
    events: the calls then run back to back on the GPU, whatever the host
    side of each call costs, which is what short launches need (from an
    eager loop the host's per-call cost can exceed the kernel's time)."""
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    cur.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fn()
    t_end = time.perf_counter() + warm_seconds
    while time.perf_counter() < t_end:
        graph.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    for _ in range(replays):
        graph.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * replays)


HEADLINE_WARM_S = 0.6
CLOCK_WINDOW_TICKS = 2_500_000       # 25 ms of the 100 MHz real-time counter


def shader_clock_under(fn, torch, iofa, dev, launches=200):
    """The shader clock while ``fn``'s kernels run back to back: ``launches``
    calls (about 50 ms at the headline workload) are queued on the current
    stream, then the clock probe (one sleeping wave, built as
    _lib/libiofa_clock.so) is started on a side stream for a 25 ms window
    that those calls cover.  Runs after the headline timing, so it does not
    share the GPU with the timed steps.  Returns None when the probe library
    is missing."""
    import ctypes
    path = os.path.join(os.path.dirname(iofa.library_path()), "libiofa_clock.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.iofa_clock_probe.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p]
    lib.iofa_clock_probe.restype = ctypes.c_int
    out = torch.zeros(2, dtype=torch.int64, device=dev)
    side = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()
    for _ in range(launches):
        fn()
    # the side stream does not wait for those calls: the probe runs beside them
    st = lib.iofa_clock_probe(ctypes.c_void_p(out.data_ptr()), CLOCK_WINDOW_TICKS,
                              ctypes.c_void_p(side.cuda_stream))
    torch.cuda.synchronize()
    if st != 0:
        raise RuntimeError(f"clock probe failed with status {st}")
    cyc, ticks = (int(x) for x in out.cpu())
    return {"shader_clock_mhz": round(100.0 * cyc / ticks, 1) if ticks else None,
            "window_ms": round(ticks / 1e5, 2),
            "how": f"s_memtime / s_memrealtime of one sleeping wave on a side stream while "
                   f"{launches} fused launches run"}


def cpu_model():
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(q, k, v, scale, spec, o_gpu, lse_gpu, target_s):
    """Time the fp64 oracle on a bounded sample (all heads, a prefix of query
    rows sized for about ``target_s`` seconds; when the whole workload takes
    less, the whole workload computed up to 8 times) and check the GPU output
    on those rows."""
    import numpy as np
    import threadpoolctl

    import oracle
    from workloads import raw_bits

    dec = {"bf16": oracle.decode_bf16, "fp16": oracle.decode_f16, "fp32": oracle.decode_f32}
    dcd = dec[spec["dtype"]]
    q64, k64, v64 = (dcd(raw_bits(t)) for t in (q, k, v))
    B, H, N, d = spec["B"], spec["H"], spec["N"], spec["d"]
    # probe: 64 rows of every head
    probe_rows = np.arange(min(64, N))
    t0 = time.perf_counter()
    oracle.standard_attention_rows(q64, k64, v64, scale, probe_rows)
    t_probe = time.perf_counter() - t0
    rows_n = int(min(N, max(64, 64 * target_s / max(t_probe, 1e-3))))
    rows = np.arange(rows_n)
    reps = 1
    if rows_n == N:
        est = t_probe * N / len(probe_rows)
        reps = int(max(1, min(8, round(target_s / max(est, 1e-3)))))
    t0 = time.perf_counter()
    for _ in range(reps):
        o_ref, lse_ref = oracle.standard_attention_rows(q64, k64, v64, scale, rows)
    t = time.perf_counter() - t0
    flops = 4.0 * B * H * rows_n * N * d * reps
    blas = [x for x in threadpoolctl.threadpool_info() if x.get("user_api") == "blas"]
    threads = blas[0]["num_threads"] if blas else 1
    o64 = dcd(raw_bits(o_gpu[:, :, :rows_n].cpu().contiguous()))
    diff = o64 - o_ref
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"all {B * H} heads, query rows 0..{rows_n - 1} of {N} "
                  f"({rows_n / N:.1%} of the workload's FLOPs)"
                  + (f", computed {reps} times" if reps > 1 else "") + ", fp64 numpy/OpenBLAS",
        "repetitions": reps,
        "seconds": round(t, 3),
        "cpu_model": cpu_model(),
        "cores_note": "BLAS threads of the fp64 products; the oracle's elementwise steps "
                      "run on one thread",
        "host_cores_visible": len(os.sched_getaffinity(0)),
        "sample_parity": {
            "max_abs": float(np.abs(diff).max()),
            "rel_f": float(np.linalg.norm(diff) / np.linalg.norm(o_ref)),
            "lse_max_abs": float(np.abs(lse_gpu[:, :, :rows_n].cpu().double().numpy()
                                        - lse_ref).max()),
        },
    }


def splitkv_contrast(spec, args, torch, iofa, dev):
    """One GPU's share of the workload when its heads are split over 8 GPUs
    (H/8 heads): few query-tile workgroups, so the key sweep is split into
    ranges and merged.  Times the fused kernel alone, the split-KV path
    (partial pass + merge) and the merge kernel alone (HBM-bound: it reads
    G*(d+1) and writes d elements + 1 fp32 LSE per row)."""
    from workloads import make_qkv
    B, H, N, d = spec["B"], max(1, spec["H"] // 8), spec["N"], spec["d"]
    q, k, v = (t.to(dev) for t in make_qkv(B, H, N, d, spec["dtype"], seed_base=4242))
    scale = iofa.default_scale(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    g = iofa.fa_splitkv_num_splits(B, H, N, d, q.dtype, 0)
    ws = torch.empty(max(16, iofa.fa_splitkv_workspace_bytes(B, H, N, d, q.dtype, g)),
                     dtype=torch.uint8, device=dev)
    flops = 4.0 * B * H * N * N * d
    f_ms = time_graph(lambda: iofa.fa_fwd(q, k, v, o, lse, scale), torch)
    share = f"{spec['dtype']} B{B} H{H} N{N} d{d} (one GPU's share of an 8-way head split)"
    if g == 1:
        # too few key tiles per range for a split to pay: the call is fa_fwd
        return {"workload": share, "num_splits": 1,
                "timing": "20 calls captured in a graph, replayed 10 times between two events",
                "fused_ms": round(f_ms, 4),
                "fused_tflops": round(flops / (f_ms * 1e-3) / 1e12, 1)}
    s_ms = time_graph(lambda: iofa.fa_fwd_splitkv(q, k, v, o, lse, ws, scale, g), torch)
    rows = B * H * N
    flat = ws.view(torch.float32)
    o_part = flat[:g * rows * d].view(g, rows, d)
    lse_part = flat[g * rows * d:g * rows * (d + 1)].view(g, rows)
    o2 = torch.empty((rows, d), dtype=q.dtype, device=dev)
    l2 = torch.empty((rows,), dtype=torch.float32, device=dev)
    m_ms = time_graph(lambda: iofa.fa_merge_partials(o_part, lse_part, o2, l2), torch)
    merge_bytes = g * rows * (d + 1) * 4 + rows * (d * q.element_size() + 4)
    return {
        "workload": share,
        "num_splits": g,
        "timing": "20 calls captured in a graph, replayed 10 times between two events",
        "fused_ms": round(f_ms, 4), "fused_tflops": round(flops / (f_ms * 1e-3) / 1e12, 1),
        "splitkv_ms": round(s_ms, 4), "splitkv_tflops": round(flops / (s_ms * 1e-3) / 1e12, 1),
        "speedup_splitkv_over_fused": round(f_ms / s_ms, 3),
        "merge_ms": round(m_ms, 4),
        "merge_roofline": {"bound": "hbm", "achieved": round(merge_bytes / (m_ms * 1e-3) / 1e9, 1),
                           "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(merge_bytes / (m_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                           "bytes_per_launch": merge_bytes},
    }


# K and V bytes the decode calls rotate over: twice the 256 MB last-level cache
DECODE_ROTATION_BYTES = 512 << 20


def decode_measure(spec, torch, iofa, dev):
    """Decode on the workload's heads: one query row per head against its N
    keys (B, H, d and dtype of the workload), through the split-KV forward
    for queries and keys of different lengths.  Bound by HBM: algorithmic
    bytes are K and V read once, Q read and O, LSE written; the partials'
    round trip through the workspace is reported beside them.

    K and V fit the 256 MB last-level cache at small sizes, and a call that
    reads the previous call's K and V would then be timed against that cache
    instead of HBM.  The calls therefore rotate over copies of K and V (equal
    values at different addresses) that together hold at least 512 MiB."""
    from workloads import make_qkv
    B, H, Nk, d = spec["B"], spec["H"], spec["N"], spec["d"]
    Nq = 1
    q = make_qkv(B, H, Nq, d, spec["dtype"], seed_base=5151)[0].to(dev)
    _, k, v = (t.to(dev) for t in make_qkv(B, H, Nk, d, spec["dtype"], seed_base=5252))
    kv_bytes = 2 * k.numel() * k.element_size()
    copies = max(1, -(-DECODE_ROTATION_BYTES // kv_bytes))
    kvs = [(k, v)] + [(k.clone(), v.clone()) for _ in range(copies - 1)]
    scale = iofa.default_scale(d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    g = iofa.fa_splitkv_qk_num_splits(B, H, Nq, Nk, d, q.dtype, 0)
    nbytes = iofa.fa_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, q.dtype, g)
    ws = torch.empty(max(16, nbytes), dtype=torch.uint8, device=dev)
    turn = [0]

    def call():
        kc, vc = kvs[turn[0] % copies]
        turn[0] += 1
        iofa.fa_fwd_splitkv_qk(q, kc, vc, o, lse, ws, scale, g)

    ms = time_graph(call, torch)
    e = q.element_size()
    alg = e * B * H * (2 * Nk * d + 2 * Nq * d) + 4 * B * H * Nq
    gbs = alg / (ms * 1e-3) / 1e9
    return {
        "workload": (f"{spec['dtype']} B{B} H{H} Nq{Nq} Nk{Nk} d{d} "
                     "(decode: one query row per head)"),
        "num_splits": g,
        "timing": ("20 calls captured in a graph, replayed 10 times between two events; "
                   f"the calls rotate over {copies} copies of K and V "
                   f"({copies * kv_bytes / 2**20:.0f} MiB)"),
        "ms": round(ms, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes": alg},
        "partials_round_trip_bytes": 2 * nbytes,
    }


# Shapes (B, H, Nq, Nk, d) and split counts of the split-count sweep
SWEEP_FULL = [(2, 2, 4096, 4096, 128), (1, 1, 16384, 16384, 128), (2, 4, 2048, 2048, 128),
              (1, 4, 8192, 8192, 128), (4, 2, 1024, 1024, 128)]
SWEEP_FULL_G = [1, 2, 3, 4, 6, 8, 12, 16]
SWEEP_DECODE = [(2, 16, 1, 4096, 128), (2, 16, 4, 4096, 128), (2, 16, 64, 4096, 128),
                (1, 32, 1, 16384, 128), (8, 32, 1, 8192, 128), (8, 32, 1, 1024, 128),
                (1, 8, 1, 32768, 128), (2, 16, 1, 1024, 128), (2, 16, 1, 512, 128),
                (1, 8, 1, 4096, 128), (1, 8, 1, 1024, 128), (1, 32, 1, 2048, 128),
                (2, 16, 1, 4096, 64), (2, 16, 1, 512, 64), (1, 8, 1, 4096, 64),
                (1, 8, 1, 1024, 64), (1, 32, 1, 2048, 64), (4, 32, 1, 2048, 64)]
SWEEP_DECODE_G = [1, 2, 4, 8, 16, 32, 64]
SWEEP_FILE = "profiles/splitkv_sweep_bf16.md"


def sweep_splits(torch, iofa, dev):
    """Time fa_fwd_splitkv_qk at every split count of the sweep lists (bf16,
    graphs of 20 calls rotating over copies of K and V that hold at least
    DECODE_ROTATION_BYTES) and write the tables, with the split count the
    library picks, to SWEEP_FILE."""
    from workloads import make_qkv

    def table(shapes, gs, title):
        rows = [f"## {title}", "",
                "| B H Nq Nk d | " + " | ".join(f"G={g}" for g in gs) + " | policy |",
                "|---" * (len(gs) + 2) + "|"]
        for (B, H, Nq, Nk, d) in shapes:
            q = make_qkv(B, H, Nq, d, "bf16", seed_base=7001)[0].to(dev)
            _, k, v = (t.to(dev) for t in make_qkv(B, H, Nk, d, "bf16", seed_base=7002))
            kv_bytes = 2 * k.numel() * k.element_size()
            copies = max(1, -(-DECODE_ROTATION_BYTES // kv_bytes))
            kvs = [(k, v)] + [(k.clone(), v.clone()) for _ in range(copies - 1)]
            o = torch.empty_like(q)
            lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
            scale = iofa.default_scale(d)
            times = {}
            auto = iofa.fa_splitkv_qk_num_splits(B, H, Nq, Nk, d, q.dtype, 0)
            for g in gs + [auto]:
                gg = iofa.fa_splitkv_qk_num_splits(B, H, Nq, Nk, d, q.dtype, g)
                if gg in times:           # capped at the key-tile count, or timed
                    continue
                nbytes = iofa.fa_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, q.dtype, gg)
                ws = torch.empty(max(16, nbytes), dtype=torch.uint8, device=dev)
                turn = [0]

                def call(gg=gg, ws=ws, turn=turn):
                    kc, vc = kvs[turn[0] % copies]
                    turn[0] += 1
                    iofa.fa_fwd_splitkv_qk(q, kc, vc, o, lse, ws, scale, gg)

                times[gg] = time_graph(call, torch) * 1e3
            best = min(times.values())
            cells = [("—" if g not in times else
                      (f"**{times[g]:.1f}**" if times[g] <= best * 1.005 else f"{times[g]:.1f}"))
                     for g in gs]
            rows.append(f"| {B} {H} {Nq} {Nk} {d} | " + " | ".join(cells) +
                        f" | {auto} ({times[auto] / best:.2f}× the fastest) |")
            print(f"[bench] sweep {B} {H} {Nq} {Nk} {d}: policy G={auto}", file=sys.stderr,
                  flush=True)
            del kvs
        return rows + [""]

    lines = ["# Split-count sweep of the split-KV forward, bf16", "",
             "Command (one MI355X, from the repository root):", "", "```",
             "python bench.py --sweep-splits", "```", "",
             "Microseconds per call of `fa_fwd_splitkv_qk` at each requested split count G: "
             "20 calls captured in a graph and replayed 10 times between two events, the calls "
             f"rotating over copies of K and V that together hold at least "
             f"{DECODE_ROTATION_BYTES >> 20} MiB, so every call reads K and V from HBM. Bold: "
             "within 0.5% of the fastest. policy: the G the library picks on its own, and its "
             "time over the fastest. A dash: G above the key-tile count (the call uses fewer).",
             ""]
    lines += table(SWEEP_FULL, SWEEP_FULL_G, "Query blocks of at least one tile (Nq = Nk)")
    lines += table(SWEEP_DECODE, SWEEP_DECODE_G, "Query blocks shorter than one tile (decode)")
    with open(SWEEP_FILE, "w", encoding="utf-8") as fh:
        fh.write("\n".join(lines))
    print(f"[bench] wrote {SWEEP_FILE}", file=sys.stderr, flush=True)


def backward_measure(q, k, v, scale, spec, args, torch, iofa, dev):
    """The backward pass on the same workload.  TFLOP/s on the algorithmic
    count 10*B*H*N^2*d (the five N^2 d products a single pass needs, 2.5x the
    forward's 4*B*H*N^2*d); the kernels recompute two more products, so they
    execute 14*B*H*N^2*d."""
    B, H, N, d = spec["B"], spec["H"], spec["N"], spec["d"]
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = iofa.forward(qd, kd, vd, scale)
    g = torch.Generator(device=dev).manual_seed(17)
    do = torch.randn(qd.shape, generator=g, device=dev).to(qd.dtype)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ws = torch.empty(iofa.fa_bwd_workspace_bytes(B, H, N), dtype=torch.uint8, device=dev)
    steps = max(5, min(args.steps, 30))
    _, ms, *_ = time_launches(lambda: iofa.fa_bwd(qd, kd, vd, o, do, lse, dq, dk, dv, ws, scale),
                          steps, 3, torch, warm_seconds=0.3)
    alg = 10.0 * B * H * N * N * d
    return {"workload": spec["name"], "ms": round(ms, 4),
            "tflops_algorithmic": round(alg / (ms * 1e-3) / 1e12, 1),
            "tflops_executed": round(1.4 * alg / (ms * 1e-3) / 1e12, 1),
            "frac_of_peak_algorithmic": round(alg / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def fp8_measure(spec, args, torch, iofa, dev):
    """The FP8 (E4M3) forward on the workload's shape: inputs from
    make_qkv_fp8 (per-tensor scales), output bf16.  TFLOP/s at 4*B*H*N^2*d
    against the dense fp8 MFMA peak."""
    from workloads import make_qkv_fp8, default_scale
    B, H, N, d = spec["B"], spec["H"], spec["N"], spec["d"]
    (q8, k8, v8), (sq, sk, sv) = make_qkv_fp8(B, H, N, d, seed_base=1000 * args.workload)
    q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    scale = default_scale(d)
    steps = max(5, min(args.steps, 50))
    _, ms, *_ = time_launches(lambda: iofa.fa_fwd_fp8(q8, k8, v8, o, lse, scale, sq, sk, sv),
                          steps, min(args.warmup, 5), torch, warm_seconds=0.3)
    tf = 4.0 * B * H * N * N * d / (ms * 1e-3) / 1e12
    return {"workload": f"fp8 (E4M3, per-tensor scales) B{B} H{H} N{N} d{d}, bf16 output",
            "ms": round(ms, 4), "tflops": round(tf, 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4)}}


def device_info(torch, dev):
    """What the runtime reports for the device the run used."""
    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1),
            "hip_runtime": getattr(torch.version, "hip", None)}


def mfma_ceiling():
    """Run the standalone MFMA-ceiling program (a child process) and return
    its cases: the sustained bf16 and fp8 MFMA rates of the whole chip at the
    fused kernels' occupancy, with the shader clock they ran at."""
    import subprocess
    exe = os.path.join(ROOT, "io_aware_softmax_04_amd", "_lib", "mfma_ceiling")
    if not os.path.exists(exe):
        return None
    proc = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                          timeout=120)
    if proc.returncode != 0:
        raise RuntimeError(f"mfma_ceiling failed: {proc.stderr.strip()}")
    return [json.loads(ln) for ln in proc.stdout.splitlines() if ln.startswith("{")]


def ceiling_cases(lines):
    """Split the ceiling program's lines into its measured cases and the
    device properties it reports first."""
    cases = [c for c in lines if "case" in c]
    props = next((c for c in lines if "device" in c), None)
    return cases, props


def softmax_measure(args, torch, iofa, dev):
    """The standalone row softmax on bf16 rows that fit one workgroup, on
    rows of 4 slices (the one-pass resident form) and on rows of 256 slices
    (two passes: x read twice), 512 MiB of x each.  Roofline: HBM;
    algorithmic bytes = read x once + write y once + 4 bytes of LSE per
    row; x_reads is what the library reports for the call."""
    out = []
    for rows, n in ((32768, 8192), (4096, 1 << 16), (64, 1 << 22)):
        g = torch.Generator(device=dev).manual_seed(rows)
        x = (torch.randn((rows, n), generator=g, device=dev) * 4).to(torch.bfloat16)
        y = torch.empty_like(x)
        lse = torch.empty(rows, dtype=torch.float32, device=dev)
        nb = iofa.fa_softmax_workspace_bytes(rows, n, x.dtype)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
        steps = max(5, min(args.steps, 30))
        wall, ms, *_ = time_launches(lambda: iofa.fa_softmax_rows(x, y, lse, ws if nb else None),
                                     steps, 3, torch, warm_seconds=0.3)
        alg = rows * n * 2 * 2 + rows * 4
        reads = iofa.fa_softmax_x_reads(x, y)
        moved = rows * n * 2 * (reads + 1) + rows * 4
        gbs = alg / (ms * 1e-3) / 1e9
        out.append({
            "workload": f"bf16 rows={rows} n={n}", "ms": round(ms, 4),
            "x_reads": reads,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes": alg},
            "moved_bytes_per_s_GBs": round(moved / (ms * 1e-3) / 1e9, 1),
            # calls back to back (no event between them): the rate a stream
            # of calls sees; a multi-kernel call loses its launch gaps there
            "ms_back_to_back": round(wall, 4),
            "frac_back_to_back": round(alg / (wall * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        })
        del x, y, ws
    return out


def main():
    args = parse()
    if args.sq_from:
        from workloads import WORKLOADS
        summarise_sq(args.sq_from, args.workload, WORKLOADS[args.workload], args.sq_kernel)
        return
    if args.trace_from:
        from workloads import WORKLOADS
        summarise_trace(args.trace_from, args.workload, WORKLOADS[args.workload], args.trace_cmd)
        return
    if args.traffic_from:
        from workloads import WORKLOADS
        summarise_traffic(args.traffic_from[0], args.traffic_from[1], args.copy_mib,
                          args.workload, WORKLOADS[args.workload])
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path shards by "
              "heads with no communication and is measured on one GPU's share.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import io_aware_softmax_04_amd as iofa
    from workloads import workload_qkv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if not os.path.exists(iofa.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    iofa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sweep_splits:
        sweep_splits(torch, iofa, dev)
        return

    q, k, v, scale, spec = workload_qkv(args.workload)
    B, H, N, d = spec["B"], spec["H"], spec["N"], spec["d"]
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    flops = 4.0 * B * H * N * N * d

    def fused():
        iofa.fa_fwd(qd, kd, vd, o, lse, scale)

    print(f"[bench] workload {args.workload}: {spec['name']}", file=sys.stderr, flush=True)
    # the timed steps start only after at least HEADLINE_WARM_S of sustained
    # launches, whatever --warmup asks for, so they see the settled clock
    wall_ms, ev_ms, ev_med, ev_min = time_launches(fused, args.steps, args.warmup, torch,
                                                   warm_seconds=HEADLINE_WARM_S)
    print(f"[bench] fused: {wall_ms:.4f} ms/step wall, {ev_ms:.4f} ms/launch (events; "
          f"median {ev_med:.4f}, min {ev_min:.4f})", file=sys.stderr, flush=True)
    achieved = flops / (ev_ms * 1e-3) / 1e12
    value = flops / (wall_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if spec["dtype"] in ("bf16", "fp16") else 157.3

    traffic = read_traffic(spec)
    clock = shader_clock_under(fused, torch, iofa, dev)
    if clock is not None:
        clock["achieved_over_peak_at_that_clock"] = round(
            flops / (ev_ms * 1e-3) / 1e12 / (PEAK_BF16_TFLOPS * clock["shader_clock_mhz"] / 2400.0),
            4) if spec["dtype"] != "fp32" else None

    models = bytes_models(spec)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec["dtype"],
        "data": "synthetic (seeded N(0,1) tensors, no dataset)",
        "config": {"workload": spec["name"], "B": B, "H": H, "N": N, "d": d,
                   "causal": False, "scale": scale, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic},
        "fused_launch_ms": round(ev_ms, 5),
        "fused_launch_ms_median": round(ev_med, 5),
        "fused_launch_ms_min": round(ev_min, 5),
        "fused_tflops_at_median": round(flops / (ev_med * 1e-3) / 1e12, 2),
        "shader_clock": clock,
        "device": device_info(torch, dev),
        "bytes_models": models,
    }

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = n * 4

    if not args.no_naive and N <= 32768:
        nb = iofa.fa_naive_workspace_bytes(B, H, N, q.dtype)
        free = torch.cuda.mem_get_info(dev)[0]
        if 2 * nb + (1 << 30) < free:
            s_ws = torch.empty(nb, dtype=torch.uint8, device=dev)
            p_ws = torch.empty(nb, dtype=torch.uint8, device=dev)
            o2 = torch.empty_like(qd)
            lse2 = torch.empty_like(lse)

            def naive():
                iofa.fa_naive_fwd(qd, kd, vd, o2, lse2, s_ws, p_ws, scale)

            nsteps = max(3, min(args.steps, 20))
            n_wall, n_ev, *_ = time_launches(naive, nsteps, min(args.warmup, 3), torch,
                                         warm_seconds=0.3)
            line["naive_contrast"] = {
                "ms_per_call": round(n_ev, 4),
                "tflops_equiv": round(flops / (n_ev * 1e-3) / 1e12, 2),
                "speedup_fused_over_naive": round(n_ev / ev_ms, 2),
                "bytes_model": models["naive_model"],
                "model_bytes_per_s_GBs": round(models["naive_model"] / (n_ev * 1e-3) / 1e9, 1),
            }
            del s_ws, p_ws
            print(f"[bench] naive: {n_ev:.4f} ms/call", file=sys.stderr, flush=True)

    if not args.no_splitkv and spec["dtype"] != "fp32":
        line["splitkv_contrast"] = splitkv_contrast(spec, args, torch, iofa, dev)
        print(f"[bench] split-KV: {line['splitkv_contrast']}", file=sys.stderr, flush=True)

    if not args.no_decode and spec["dtype"] != "fp32":
        line["decode"] = decode_measure(spec, torch, iofa, dev)
        print(f"[bench] decode: {line['decode']}", file=sys.stderr, flush=True)

    if not args.no_backward and spec["dtype"] != "fp32":
        line["backward"] = backward_measure(q, k, v, scale, spec, args, torch, iofa, dev)
        print(f"[bench] backward: {line['backward']}", file=sys.stderr, flush=True)

    if not args.no_fp8 and spec["dtype"] != "fp32":
        line["fp8_forward"] = fp8_measure(spec, args, torch, iofa, dev)
        print(f"[bench] fp8 forward: {line['fp8_forward']}", file=sys.stderr, flush=True)

    if not args.no_softmax:
        line["softmax_rows"] = softmax_measure(args, torch, iofa, dev)
        print(f"[bench] row softmax: {line['softmax_rows']}", file=sys.stderr, flush=True)

    if not args.no_ceiling:
        cases, props = ceiling_cases(mfma_ceiling() or [])
        if props:
            line["device"]["hip_properties"] = props
        if cases:
            rnd = [c for c in cases if c["case"].startswith("bf16") and "random" in c["case"]]
            line["mfma_ceiling"] = {"cases": cases}
            if rnd:
                line["mfma_ceiling"]["fused_frac_of_bf16_random_ceiling"] = round(
                    achieved / rnd[0]["tflops"], 4)
            ex = [c for c in cases if c["case"].startswith("v_exp_f32")]
            if ex:
                # one exponential per score: B*H*N^2 of them at the chip's
                # measured v_exp_f32 rate is a floor under the fused kernel
                n_exp = float(B * H * N * N)
                floor_ms = n_exp / ex[0]["lane_ops_per_s"] * 1e3
                line["exp_floor"] = {"exponentials": n_exp,
                                     "rate_per_s": ex[0]["lane_ops_per_s"],
                                     "ms": round(floor_ms, 4),
                                     "frac_of_fused_launch": round(floor_ms / ev_ms, 4)}
            print(f"[bench] MFMA ceiling: {line['mfma_ceiling']}", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on a bounded sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(q, k, v, scale, spec, o, lse, args.cpu_seconds)

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
