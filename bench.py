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
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd attention TFLOP/s (4BHN²d/t) + % bf16 MFMA peak, N=4096 d=128"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16/fp16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
FUSED_KERNEL_SOURCES = ["io_aware_softmax_04_amd/csrc/fa_fwd_gfx950.hip",
                        "io_aware_softmax_04_amd/csrc/fa_device.h"]
TRAFFIC_FILE = "profiles/traffic_fused_fwd_{tag}.json"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", type=int, default=3)
    p.add_argument("--no-naive", action="store_true", help="skip the naive contrast")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="also run a device copy of this many MiB (counter calibration)")
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


def time_launches(fn, steps, warmup, torch):
    """Run ``fn`` warmup + steps times; returns (wall ms per step, mean launch
    ms from HIP events recorded on the launch stream around each call)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ev = sum(a.elapsed_time(b) for a, b in evs) / steps
    return wall, ev


def cpu_baseline(q, k, v, scale, spec, o_gpu, lse_gpu, target_s):
    """Time the fp64 oracle on a bounded sample (all heads, a prefix of query
    rows sized for about ``target_s`` seconds) and check the GPU output on
    those rows."""
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
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.standard_attention_rows(q64, k64, v64, scale, rows)
    t = time.perf_counter() - t0
    flops = 4.0 * B * H * rows_n * N * d
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
                  f"({rows_n / N:.1%} of the workload's FLOPs), fp64 numpy/OpenBLAS",
        "seconds": round(t, 3),
        "host_cores_visible": len(os.sched_getaffinity(0)),
        "sample_parity": {
            "max_abs": float(np.abs(diff).max()),
            "rel_f": float(np.linalg.norm(diff) / np.linalg.norm(o_ref)),
            "lse_max_abs": float(np.abs(lse_gpu[:, :, :rows_n].cpu().double().numpy()
                                        - lse_ref).max()),
        },
    }


def main():
    args = parse()
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

    q, k, v, scale, spec = workload_qkv(args.workload)
    B, H, N, d = spec["B"], spec["H"], spec["N"], spec["d"]
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    flops = 4.0 * B * H * N * N * d

    def fused():
        iofa.fa_fwd(qd, kd, vd, o, lse, scale)

    print(f"[bench] workload {args.workload}: {spec['name']}", file=sys.stderr, flush=True)
    wall_ms, ev_ms = time_launches(fused, args.steps, args.warmup, torch)
    print(f"[bench] fused: {wall_ms:.4f} ms/step wall, {ev_ms:.4f} ms/launch (events)",
          file=sys.stderr, flush=True)
    achieved = flops / (ev_ms * 1e-3) / 1e12
    value = flops / (wall_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if spec["dtype"] in ("bf16", "fp16") else 157.3

    traffic = None
    tpath = os.path.join(ROOT, TRAFFIC_FILE.format(tag=workload_tag(spec)))
    if os.path.exists(tpath):
        with open(tpath, encoding="utf-8") as fh:
            rec = json.load(fh)
        if rec.get("kernel_sources_sha256_16") == sources_hash():
            traffic = rec.get("bytes_per_launch")

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
            n_wall, n_ev = time_launches(naive, nsteps, min(args.warmup, 3), torch)
            line["naive_contrast"] = {
                "ms_per_call": round(n_ev, 4),
                "tflops_equiv": round(flops / (n_ev * 1e-3) / 1e12, 2),
                "speedup_fused_over_naive": round(n_ev / ev_ms, 2),
                "bytes_model": models["naive_model"],
                "model_bytes_per_s_GBs": round(models["naive_model"] / (n_ev * 1e-3) / 1e9, 1),
            }
            del s_ws, p_ws
            print(f"[bench] naive: {n_ev:.4f} ms/call", file=sys.stderr, flush=True)

    if not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on a bounded sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(q, k, v, scale, spec, o, lse, args.cpu_seconds)

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
