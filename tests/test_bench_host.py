"""Host-side logic of bench.py that needs no GPU: the algorithmic byte
models, the launch grid that tells the fused kernel's dispatches apart in a
trace, the split of the ceiling program's output, and the one-GPU guard."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import WORKLOADS  # noqa: E402


# Per workload: compulsory bytes e*4Nd + 4N per head (Q, K, V read once, O and
# the fp32 LSE written once), the tiled-IO model e*(2Nd + 2Nd*ceil(N/128)) + 4N
# per head (K and V streamed once per 128-row query tile) and the naive model
# e*(4Nd + 4N^2) per head (the element count of the three-step standard
# attention, S and P stored in the input type).  Worked out by hand from those
# definitions for each workload's shape.
EXPECTED = {
    1: (263_168, 394_240, 1_310_720),
    2: (33_816_576, 151_257_088, 570_425_344),
    3: (134_742_016, 2_215_116_800, 4_429_185_024),
    4: (538_968_064, 34_630_270_976, 69_256_347_648),
    5: (134_725_568, 4_362_067_904, 8_722_038_912),
}


@pytest.mark.parametrize("idx", sorted(EXPECTED))
def test_byte_models(idx):
    m = bench.bytes_models(WORKLOADS[idx])
    assert (m["compulsory"], m["tiled_io_model"], m["naive_model"]) == EXPECTED[idx]


def test_byte_models_order():
    # the tiled model never undercuts the compulsory bytes, and the naive
    # model exceeds the tiled one whenever N is above the query tile
    for spec in WORKLOADS.values():
        m = bench.bytes_models(spec)
        assert m["compulsory"] <= m["tiled_io_model"] <= m["naive_model"]


def test_fused_grid_of_the_benchmark_workload():
    # d = 128: B*H*ceil(N/256) workgroups of 512 work-items, 512 workgroups at
    # B2 H16 N4096, the grid the kernel trace lists for the fused forward;
    # d = 64: B*H*ceil(N/128) workgroups of 256
    assert bench.fused_grid_items(WORKLOADS[3]) == 512 * 512
    assert bench.fused_grid_items(WORKLOADS[5]) == 2 * 8 * 32 * 512
    assert bench.fused_grid_items(WORKLOADS[2]) == 4 * 16 * 8 * 256


def test_ceiling_output_split():
    lines = [{"device": "X", "max_shader_clock_mhz": 2400},
             {"case": "bf16 32x32x16, constant operands", "tflops": 1.0},
             {"case": "v_exp_f32, 8 chains per lane", "lane_ops_per_s": 2.0}]
    cases, props = bench.ceiling_cases(lines)
    assert [c["case"] for c in cases] == [lines[1]["case"], lines[2]["case"]]
    assert props == lines[0]
    assert bench.ceiling_cases([]) == ([], None)


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                          timeout=120, cwd=ROOT)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr
    assert proc.stdout == ""


def _fake_trace(directory, fused_ns, other_ns):
    # the columns of rocprofv3's kernel_trace.csv that the summary reads
    spec = WORKLOADS[3]
    grid = bench.fused_grid_items(spec)
    rows = ["Kernel_Name,Grid_Size_X,Grid_Size_Y,Grid_Size_Z,Start_Timestamp,End_Timestamp"]
    t = 1000
    for ns in fused_ns:
        rows.append(f'"void iofa::fa_fwd_16_kernel<iofa::Bf16, 128, 32, false, 8>(...)",'
                    f'{grid},1,1,{t},{t + ns}')
        t += ns + 10
    # the split-KV partial pass of the same kernel at the same grid is not the fused forward
    rows.append(f'"void iofa::fa_fwd_16_kernel<iofa::Bf16, 128, 32, true, 8>(...)",{grid},1,1,{t},{t + 999_999}')
    t += 999_999 + 10
    for ns in other_ns:
        rows.append(f'"void iofa::naive_pv_16<iofa::Bf16, 128>(...)",1024,1,1,{t},{t + ns}')
        t += ns + 10
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "run_kernel_trace.csv"), "w") as fh:
        fh.write("\n".join(rows) + "\n")


def test_fused_rows_are_told_apart_by_name_and_grid():
    spec = WORKLOADS[3]
    grid = bench.fused_grid_items(spec)
    for name, want in (("void iofa::fa_fwd_16_kernel<iofa::Bf16, 128, 32, false, 8>(...)", True),
                       ("void iofa::fa_fwd_16_kernel<iofa::Bf16, 128, 32, false>(...)", True),
                       ("void iofa::fa_fwd_16_kernel<iofa::Bf16, 128, 32, true, 8>(...)", False),
                       ("void iofa::fa_fwd_fp8_kernel<128>(...)", False)):
        assert bench._is_fused({"Kernel_Name": name, "Grid_Size": grid}, spec) is want, name
    assert not bench._is_fused({"Kernel_Name": "void iofa::fa_fwd_16_kernel<iofa::Bf16, 128, 32, "
                                               "false, 4>(...)", "Grid_Size": grid // 8}, spec)


def test_trace_summary_quotes_the_profiled_run(tmp_path):
    # the fused rows' average (250 us here) is set against the bench line kept
    # beside the trace (250 us from events), and the rate uses 4*B*H*N^2*d
    trace = tmp_path / "kt"
    _fake_trace(str(trace), [240_000, 260_000], [90_000])
    line = {"fused_launch_ms": 0.25, "fused_launch_ms_median": 0.25,
            "roofline": {"achieved": 1099.5}}
    (trace / bench.BENCH_STDOUT).write_text("[bench] log line\n" + __import__("json").dumps(line) + "\n")
    out = tmp_path / "out"
    out.mkdir()
    path = bench.summarise_trace(str(trace), 3, WORKLOADS[3], "--no-cpu-baseline", out_dir=str(out))
    text = open(path).read()
    assert path.startswith(str(out))
    assert "| 2 | 250000 | 240000 | 260000 | 1099.5 |" in text
    assert "trace / events = 1.000" in text
    assert f"> {trace / bench.BENCH_STDOUT}" in text


def test_trace_summary_without_the_profiled_run(tmp_path):
    trace = tmp_path / "kt"
    _fake_trace(str(trace), [250_000], [])
    out = tmp_path / "out"
    out.mkdir()
    text = open(bench.summarise_trace(str(trace), 3, WORKLOADS[3], "", out_dir=str(out))).read()
    assert "trace / events" not in text
    assert bench.BENCH_STDOUT not in text


def _pmc_csv(directory, kernel, grid, values, ns, dispatches=3):
    import csv
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                           "Counter_Name", "Counter_Value", "Start_Timestamp",
                                           "End_Timestamp"])
        w.writeheader()
        for i in range(dispatches):
            for c, v in values.items():
                w.writerow({"Dispatch_Id": 10 + 2 * i, "Kernel_Name": kernel, "Grid_Size": grid,
                            "Counter_Name": c, "Counter_Value": v, "Start_Timestamp": 1000,
                            "End_Timestamp": 1000 + ns})


def test_shader_counter_summary_of_two_passes(tmp_path):
    # a kernel of 200 us at 1500 MHz: 300000 cycles per engine; MFMA busy
    # half the SIMD-cycles; waves wait a quarter of their lifetime
    cyc = 300000.0
    a = {"SQ_BUSY_CYCLES": 32 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * bench.SIMDS * cyc,
         "SQ_INSTS_VALU": 6000.0 * 4096, "SQ_INSTS_MFMA": 1000.0 * 4096, "SQ_INSTS_LDS": 500.0 * 4096,
         "SQ_INSTS_VALU_TRANS_F32": 900.0 * 4096, "SQ_WAVES": 4096.0, "SQ_WAVE_CYCLES": 4.0e8}
    b = {"SQ_BUSY_CYCLES": 32 * cyc, "SQ_WAVE_CYCLES": 4.0e8, "SQ_WAIT_ANY": 1.0e8,
         "SQ_WAIT_INST_LDS": 2.0e7, "SQ_VALU_MFMA_COEXEC_CYCLES": 0.2 * bench.SIMDS * cyc,
         "SQ_ACTIVE_INST_VALU": 0.1 * bench.SIMDS * cyc, "SQ_ACTIVE_INST_LDS": 0.05 * bench.SIMDS * cyc,
         "SQ_INSTS_SALU": 100.0 * 4096}
    name = "void iofa::bwd_dkdv_kernel<iofa::Bf16, 128>(...)"
    _pmc_csv(str(tmp_path / "a"), name, 1024, a, 200000)
    _pmc_csv(str(tmp_path / "b"), name, 1024, b, 200000)
    out = tmp_path / "out"
    out.mkdir()
    path = bench.summarise_sq([str(tmp_path / "a"), str(tmp_path / "b")], 3, WORKLOADS[3],
                              "bwd_dkdv", out_dir=str(out))
    text = open(path).read()
    assert os.path.basename(path) == "sq_counters_bwd_dkdv_bf16_B2H16N4096d128.md"
    assert "| effective shader clock | 1500 MHz" in text
    assert "| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / SIMDs / cycles) | 0.500 |" in text
    assert "(COEXEC / SIMDs / cycles) | 0.200 |" in text
    assert "(4 x ACTIVE_INST_VALU / SIMDs / cycles) | 0.400 |" in text
    assert "(WAIT_ANY / WAVE_CYCLES) | 0.250 |" in text
    assert "(WAIT_INST_LDS / WAVE_CYCLES) | 0.050 |" in text
    assert "| 1000 / 6000 / 900 / 500 |" in text
    # 1000 MFMAs per wave x 4096 waves x 32768 FLOP in 200 us
    assert f"{1000 * 4096 * 32768 / 200e-6 / 1e12:.1f} TFLOP/s" in text


def test_shader_counter_summary_with_unequal_passes(tmp_path):
    # pass a has 3 dispatches, pass b 5: each counter averages its own
    cyc = 300000.0
    a = {"SQ_BUSY_CYCLES": 32 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.4 * bench.SIMDS * cyc,
         "SQ_INSTS_VALU": 100.0, "SQ_INSTS_MFMA": 10.0, "SQ_INSTS_LDS": 5.0,
         "SQ_INSTS_VALU_TRANS_F32": 1.0, "SQ_WAVES": 1.0, "SQ_WAVE_CYCLES": 1.0e8}
    b = {"SQ_BUSY_CYCLES": 32 * cyc, "SQ_WAVE_CYCLES": 1.0e8, "SQ_WAIT_ANY": 3.0e7,
         "SQ_WAIT_INST_LDS": 1.0e7, "SQ_VALU_MFMA_COEXEC_CYCLES": 0.1 * bench.SIMDS * cyc,
         "SQ_ACTIVE_INST_VALU": 0.1 * bench.SIMDS * cyc,
         "SQ_ACTIVE_INST_LDS": 0.1 * bench.SIMDS * cyc, "SQ_INSTS_SALU": 7.0}
    name = "void iofa::(anonymous namespace)::fa_fwd_fp8_kernel<128>(...)"
    _pmc_csv(str(tmp_path / "a"), name, 1024, a, 150000, dispatches=3)
    _pmc_csv(str(tmp_path / "b"), name, 1024, b, 150000, dispatches=5)
    out = tmp_path / "out"
    out.mkdir()
    text = open(bench.summarise_sq([str(tmp_path / "a"), str(tmp_path / "b")], 3, WORKLOADS[3],
                                   "fp8", out_dir=str(out))).read()
    assert "| 0.400 |" in text and "(WAIT_ANY / WAVE_CYCLES) | 0.300 |" in text
    assert "| 10 / 100 / 1 / 5 |" in text


def test_shader_counter_summary_with_the_lds_pass(tmp_path):
    # 300000 cycles; the LDS returns 2^33 bytes in 2^25 active cycles summed
    # over the CUs: 256 bytes per active cycle, busy 2^25 / (256 x 300000)
    cyc = 300000.0
    a = {"SQ_BUSY_CYCLES": 32 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * bench.SIMDS * cyc,
         "SQ_INSTS_VALU": 100.0, "SQ_INSTS_MFMA": 10.0, "SQ_INSTS_LDS": 5.0,
         "SQ_INSTS_VALU_TRANS_F32": 1.0, "SQ_WAVES": 1.0, "SQ_WAVE_CYCLES": 1.0e8}
    b = {"SQ_BUSY_CYCLES": 32 * cyc, "SQ_WAVE_CYCLES": 1.0e8, "SQ_WAIT_ANY": 3.0e7,
         "SQ_WAIT_INST_LDS": 1.0e7, "SQ_VALU_MFMA_COEXEC_CYCLES": 0.1 * bench.SIMDS * cyc,
         "SQ_ACTIVE_INST_VALU": 0.1 * bench.SIMDS * cyc,
         "SQ_ACTIVE_INST_LDS": 0.1 * bench.SIMDS * cyc, "SQ_INSTS_SALU": 7.0}
    c = {"SQ_BUSY_CYCLES": 32 * cyc, "SQ_INSTS_LDS": 5.0, "SQ_INSTS_LDS_LOAD_BANDWIDTH": 2.0 ** 27,
         "SQ_LDS_IDX_ACTIVE": 2.0 ** 25, "SQ_LDS_BANK_CONFLICT": 2.0 ** 23,
         "SQ_LDS_ADDR_CONFLICT": 0.0, "SQ_LDS_CMD_FIFO_FULL": 2.0 ** 15,
         "SQ_LDS_DATA_FIFO_FULL": 0.0}
    assert sorted(c) == sorted(bench.SQ_PASSES["c"])
    name = "void iofa::bwd_dq_kernel<iofa::Bf16, 128>(...)"
    for k, v in (("a", a), ("b", b), ("c", c)):
        _pmc_csv(str(tmp_path / k), name, 1024, v, 200000)
    out = tmp_path / "out"
    out.mkdir()
    text = open(bench.summarise_sq([str(tmp_path / k) for k in "abc"], 3, WORKLOADS[3],
                                   "bwd_dq", out_dir=str(out))).read()
    assert "rocprofv3 --pmc " + " ".join(bench.SQ_PASSES["c"]) in text
    assert "(64 x SQ_INSTS_LDS_LOAD_BANDWIDTH) | 8.59e+09 |" in text
    assert "(bytes / SQ_LDS_IDX_ACTIVE) | 256 |" in text
    assert f"(SQ_LDS_IDX_ACTIVE / CUs / cycles) | {2 ** 25 / (256 * cyc):.3f} |" in text
    assert "conflict cycles per active cycle | 0.250 / 0.000 |" in text
    assert "FIFO full cycles per active cycle | 0.0010 / 0.0000 |" in text


def test_traffic_calibration_sums_a_split_copy(tmp_path):
    # the 1024 MiB calibration copy ran as two dispatches of 512 MiB: the
    # scale comes from their sum, not their mean
    import csv

    def pmc(directory, counter, fused_kib, copy_kibs):
        os.makedirs(directory)
        with open(os.path.join(directory, "run_counter_collection.csv"), "w", newline="") as fh:
            w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                               "Counter_Name", "Counter_Value",
                                               "Start_Timestamp", "End_Timestamp"])
            w.writeheader()
            n = 0
            for v in copy_kibs:
                w.writerow({"Dispatch_Id": n, "Kernel_Name": bench.COPY_KERNEL_NAME, "Grid_Size": 512,
                            "Counter_Name": counter, "Counter_Value": v, "Start_Timestamp": 0,
                            "End_Timestamp": 1})
                n += 1
            for _ in range(3):
                w.writerow({"Dispatch_Id": n, "Grid_Size": bench.fused_grid_items(WORKLOADS[3]),
                            "Kernel_Name": "void iofa::fa_fwd_16_kernel<iofa::Bf16, 128, 32, false>()",
                            "Counter_Name": counter, "Counter_Value": fused_kib,
                            "Start_Timestamp": 0, "End_Timestamp": 1})
                n += 1

    # FETCH_SIZE sees half the bytes read, WRITE_SIZE all the bytes written
    pmc(str(tmp_path / "f"), "FETCH_SIZE", 49260.0, [262144.0, 262144.0])
    pmc(str(tmp_path / "w"), "WRITE_SIZE", 33280.0, [524288.0, 524288.0])
    old = bench.ROOT
    try:
        bench.ROOT = str(tmp_path)
        os.makedirs(tmp_path / "profiles")
        os.makedirs(tmp_path / "io_aware_softmax_04_amd" / "csrc")
        for rel in bench.FUSED_KERNEL_SOURCES:
            open(tmp_path / rel, "w").write("x")
        bench.summarise_traffic(str(tmp_path / "f"), str(tmp_path / "w"), 1024, 3, WORKLOADS[3])
        text = open(tmp_path / "profiles" / "traffic_fused_fwd_bf16_B2H16N4096d128.md").read()
    finally:
        bench.ROOT = old
    assert "scaled by 2.0000 (fetch) and 4.0000 (write)" not in text
    assert "scaled by 4.0000 (fetch) and 2.0000 (write)" not in text
    assert "scaled by 2.0000 (fetch) and 1.0000 (write)" in text
    assert f"bytes_per_launch: {round(49260.0 * 1024 * 2 + 33280.0 * 1024)}" in text


def test_cpu_baseline_repeats_a_whole_workload_that_finishes_early():
    # a one-head workload the oracle finishes in milliseconds: the whole of
    # it is the sample, repeated (at most 8 times) toward the target seconds
    import torch
    from workloads import make_qkv
    spec = {"B": 1, "H": 1, "N": 64, "d": 64, "dtype": "bf16"}
    q, k, v = make_qkv(1, 1, 64, 64, "bf16", seed_base=7)
    o = torch.zeros_like(q)
    lse = torch.zeros((1, 1, 64), dtype=torch.float32)
    r = bench.cpu_baseline(q, k, v, 0.125, spec, o, lse, target_s=5.0)
    assert r["repetitions"] == 8
    assert "query rows 0..63 of 64 (100.0% of the workload's FLOPs), computed 8 times" in r["sample"]
    assert r["value"] > 0 and r["seconds"] > 0
    # the parity figures compare the given output (zeros here) with the oracle's
    assert r["sample_parity"]["max_abs"] > 0
