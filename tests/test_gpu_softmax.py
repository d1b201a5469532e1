"""GPU parity of the standalone row softmax (fa_softmax_rows) against the
fp64 oracle's row softmax, through the C ABI.

Tolerance: the output is rounded once to its type (u|y|, u = 2^-24 fp32,
2^-11 fp16, 2^-8 bf16; below the smallest normal fp16 value 2^-14 the
rounding error is at most half the subnormal spacing, 2^-25, absolute), on
top of the fp32 arithmetic's relative error REL:
  fp32 outputs (accurate expf; sums of at most 16 terms per thread, then
  256-way and chunk-way merges): 4e-6;
  16-bit outputs (hardware exp2 of (x - m) log2 e + 64): the argument
  a = t log2 e + 64 (t = x - m <= 0) carries t's rounding and log2 e's
  (1.5 * 2^-24 |t| log2 e) plus the fma's (2^-24 |a|), at most
  396 * 2^-24 log2 units for |t| <= 92; times ln 2 that is 1.64e-5
  relative, plus one ulp of v_exp_f32 and 1.2e-6 for the sums: under 2e-5
  wherever a bf16 result is above its smallest subnormal (|t| <= 92;
  smaller results fall under the absolute floor).
LSE: REL * (1 + |LSE|)."""

import numpy as np
import pytest
import torch

import io_aware_softmax_04_amd as iofa
import oracle
from helpers import UNIT_ROUNDOFF, widen

pytestmark = pytest.mark.gpu

DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
REL = {torch.float32: 4e-6, torch.float16: 2e-5, torch.bfloat16: 2e-5}
# absolute floor of the output rounding (subnormal range of the output type)
ABS_FLOOR = {torch.float32: 2.0 ** -150, torch.float16: 2.0 ** -25, torch.bfloat16: 2.0 ** -134}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    iofa.load_library()
    return torch.device("cuda:0")


def _inputs(rows, n, dtype, seed, spread=5.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((rows, n), generator=g) * spread
    if n > 1:
        x[0, n // 2] += 40.0                       # one dominant entry in row 0
        x[-1] += torch.linspace(0, 30, n)          # maximum reached late in the last row
    return x.to(DT[dtype]).contiguous()


def _check(x, y, lse, label):
    y_ref, lse_ref = oracle.softmax_rows(widen(x))
    got = widen(y.cpu())
    u = UNIT_ROUNDOFF[x.dtype]
    rel = REL[x.dtype]
    excess = np.abs(got - y_ref) - (u + rel) * np.abs(y_ref) - ABS_FLOOR[x.dtype]
    assert excess.max() <= 0, f"{label}: worst excess {excess.max():.3e}"
    if lse is not None:
        d = np.abs(lse.cpu().double().numpy() - lse_ref)
        assert np.all(d <= rel * (1 + np.abs(lse_ref))), f"{label}: lse {d.max():.3e}"


# One-chunk rows, rows that take the two passes (odd lengths: scalar
# accesses; aligned rows of more than 32 slices: 16-byte accesses) and rows
# of at most 32 slices that take the one-pass resident form, with ragged last
# slices (16392 = 2 slices + 8 elements for 16-bit types) and the 32-slice
# boundary ((1 << 19) 16-bit elements are 32 slices, 16 more are 33).
SHAPES = [(1, 1), (3, 7), (5, 100), (7, 4096), (4, 8192), (4, 8193), (2, 20001), (2, 8200),
          (5, 16392), (3, 40000), (3, 1 << 18), (2, 1 << 19), (2, (1 << 19) + 16), (2, 1 << 20)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_softmax_matches_oracle(dtype, dev):
    for rows, n in SHAPES:
        x = _inputs(rows, n, dtype, seed=rows * 7 + n)
        print(f"softmax {dtype} rows={rows} n={n}", flush=True)
        y, lse = iofa.softmax(x.to(dev), want_lse=True)
        torch.cuda.synchronize()
        _check(x, y, lse, f"{dtype} {rows}x{n}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_softmax_in_place_and_rows_sum_to_one(dtype, dev):
    # one chunk, one-pass slices, two passes with 16-byte and with scalar accesses
    for rows, n in ((6, 3000), (3, 50000), (2, 1 << 20), (3, 20001)):
        x = _inputs(rows, n, dtype, seed=n)
        xd = x.to(dev)
        nbytes = iofa.fa_softmax_workspace_bytes(rows, n, xd.dtype)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
        iofa.fa_softmax_rows(xd, xd, None, ws)          # in place
        torch.cuda.synchronize()
        _check(x, xd, None, f"in place {dtype} {rows}x{n}")
        s = xd.double().sum(dim=1).cpu().numpy()
        assert np.abs(s - 1).max() <= (2e-3 if dtype == "bf16" else 1e-5)


def test_softmax_forms_cover_every_path(dev):
    # which form the shapes above take on an idle device (the one-pass form
    # needs its grid resident at once, which an MI355X allows for 32 slices)
    def reads(rows, n, dtype):
        x = torch.empty((rows, n), dtype=DT[dtype], device=dev)
        return iofa.fa_softmax_x_reads(x, torch.empty_like(x))
    assert reads(7, 4096, "bf16") == 1
    assert reads(4, 8193, "bf16") == 2            # odd length: scalar two passes
    assert reads(2, 8200, "bf16") == 1
    assert reads(5, 16392, "fp32") == 1
    assert reads(3, 1 << 18, "bf16") == 1
    assert reads(2, 1 << 19, "bf16") == 1         # 32 slices
    assert reads(2, (1 << 19) + 16, "bf16") == 2  # 33 slices
    assert reads(2, 1 << 19, "fp32") == 2         # 64 slices of 8192
    assert reads(64, 1 << 22, "bf16") == 2


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_softmax_repair_path_matches_oracle(dtype, dev):
    # a wait bound of one poll sends every slice that finds its row
    # incomplete to the repair kernel; the results must not change
    prev = iofa.fa_softmax_set_wait_limit(0)
    try:
        for rows, n in ((3, 1 << 18), (5, 16392), (40, 100000)):
            x = _inputs(rows, n, dtype, seed=3 * rows + n)
            print(f"softmax repair {dtype} rows={rows} n={n}", flush=True)
            y, lse = iofa.softmax(x.to(dev), want_lse=True)
            torch.cuda.synchronize()
            _check(x, y, lse, f"repair {dtype} {rows}x{n}")
        x = _inputs(3, 50000, dtype, seed=17)
        xd = x.to(dev)
        ws = torch.empty(iofa.fa_softmax_workspace_bytes(3, 50000, xd.dtype), dtype=torch.uint8,
                         device=dev)
        iofa.fa_softmax_rows(xd, xd, None, ws)          # in place
        torch.cuda.synchronize()
        _check(x, xd, None, f"repair in place {dtype}")
    finally:
        iofa.fa_softmax_set_wait_limit(prev)


def test_softmax_resident_beside_a_busy_stream(dev):
    # the one-pass form needs every slice of a row resident at once; with the
    # fused forward occupying the chip from another stream that may not hold,
    # and slices whose wait runs out go to the repair kernel: the result must
    # not change
    from workloads import default_scale, make_qkv
    q, k, v = (t.to(dev) for t in make_qkv(2, 16, 4096, 128, "bf16", seed_base=808))
    o = torch.empty_like(q)
    lse_f = torch.empty((2, 16, 4096), dtype=torch.float32, device=dev)
    busy, side = torch.cuda.Stream(), torch.cuda.Stream()
    cases = [_inputs(48, 1 << 19, "bf16", seed=91), _inputs(64, 100000, "fp32", seed=92)]
    for i, x in enumerate(cases):
        xd = x.to(dev)
        y = torch.empty_like(xd)
        lse = torch.empty(xd.shape[0], dtype=torch.float32, device=dev)
        ws = torch.empty(iofa.fa_softmax_workspace_bytes(*xd.shape, xd.dtype), dtype=torch.uint8,
                         device=dev)
        assert iofa.fa_softmax_x_reads(xd, y) == 1
        torch.cuda.synchronize()
        with torch.cuda.stream(busy):
            for _ in range(20):
                iofa.fa_fwd(q, k, v, o, lse_f, default_scale(128))
        with torch.cuda.stream(side):
            for _ in range(3):
                iofa.fa_softmax_rows(xd, y, lse, ws)
        torch.cuda.synchronize()
        print(f"softmax beside a busy stream, case {i}: {tuple(xd.shape)} {xd.dtype}", flush=True)
        _check(x, y, lse, f"beside a busy stream {i}")


def test_softmax_unaligned_rows_take_the_scalar_path(dev):
    # a base one element past a 16-byte boundary and an odd row length
    buf = _inputs(1, 5 * 9001 + 1, "bf16", seed=5).view(-1).to(dev)
    x = buf[1:].view(5, 9001)
    y = torch.empty_like(x)
    lse = torch.empty(5, dtype=torch.float32, device=dev)
    ws = torch.empty(iofa.fa_softmax_workspace_bytes(5, 9001, x.dtype), dtype=torch.uint8,
                     device=dev)
    iofa.fa_softmax_rows(x, y, lse, ws)
    torch.cuda.synchronize()
    _check(x.cpu(), y, lse, "unaligned bf16 5x9001")


def test_softmax_stress_spread(dev):
    # scores of the numerics-stress attention workload scale: spread about 16
    for dtype in ("fp16", "bf16"):
        x = _inputs(8, 8191, dtype, seed=99, spread=16.0)
        y, lse = iofa.softmax(x.to(dev), want_lse=True)
        torch.cuda.synchronize()
        _check(x, y, lse, f"stress {dtype}")


@pytest.mark.parametrize("rows,n,picked", [(32768, 8192, 48), (4096, 1 << 16, 24),
                                            (64, 1 << 22, 3)])
def test_softmax_at_the_benchmarked_shapes(rows, n, picked, dev):
    # the three shapes the bench times (rows of one chunk, rows of 4 slices
    # through the one-pass form, rows of 512 chunks through the two passes),
    # in the same launch configuration;
    # rows are independent, so sampled rows (and the first and last) are held
    # to the oracle's softmax of those rows
    x = _inputs(rows, n, "bf16", seed=rows + 1, spread=4.0)
    xd = x.to(dev)
    y, lse = iofa.softmax(xd, want_lse=True)
    torch.cuda.synchronize()
    g = np.random.default_rng(rows)
    sel = np.unique(np.concatenate([[0, rows - 1], g.choice(rows, picked, replace=False)]))
    print(f"softmax bf16 {rows}x{n}: checking {sel.size} rows", flush=True)
    _check(x[sel], y.cpu()[sel], lse.cpu()[sel], f"bf16 {rows}x{n} sampled rows")
    del xd, y
