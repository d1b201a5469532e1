"""GPU parity of the fused and the naive paths against the fp64 oracle,
called through the C ABI (python binding -> libiofa.so)."""

import numpy as np
import pytest
import torch

import io_aware_softmax_04_amd as iofa
from helpers import (assert_parity, errors, naive_output_bound, nan_outputs, oracle_full,
                     oracle_rows, tile_rows, widen, workload_oracle)
from workloads import WORKLOADS, default_scale, make_qkv, workload_qkv

pytestmark = pytest.mark.gpu

DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    iofa.load_library()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _run(fn, q, k, v, scale, dev, **kw):
    out = fn(q.to(dev), k.to(dev), v.to(dev), scale, **kw)
    torch.cuda.synchronize()
    o, lse = out
    return o.cpu(), (lse.cpu() if lse is not None else None)


# ------------------------------------------------------- named workloads

@pytest.mark.parametrize("idx", sorted(WORKLOADS))
def test_fused_workload(idx, dev):
    # every element of O and LSE against the oracle, outputs NaN-filled
    # before the launch so an element the kernel never writes fails
    q, k, v, scale, spec = workload_qkv(idx)
    _say(f"fused workload {idx}: {spec['name']} scale={scale}")
    o, lse = nan_outputs(q, dev)
    iofa.fa_fwd(q.to(dev), k.to(dev), v.to(dev), o, lse, scale)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    o_ref, lse_ref = workload_oracle(idx)
    res = assert_parity(o, lse, o_ref, lse_ref, q.dtype, f"fused w{idx} (every element)")
    _say(f"  max_abs={res[0]:.3e} rel_f={res[1]:.3e} lse={res[2]:.3e}")


# ------------------------------------------------------------ ragged shapes

RAGGED_N = [1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 127, 128, 129, 255, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_fused_ragged(dtype, d, dev):
    for N in RAGGED_N:
        q, k, v = make_qkv(1, 3, N, d, dtype, seed_base=10 * N + d, dist="normal")
        scale = default_scale(d)
        _say(f"fused ragged {dtype} d={d} N={N}")
        o, lse = _run(iofa.forward, q, k, v, scale, dev)
        o_ref, lse_ref = oracle_full(q, k, v, scale)
        assert_parity(o, lse, o_ref, lse_ref, q.dtype, f"ragged {dtype} d={d} N={N}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fused_stress_distribution_small(dtype, dev):
    # scores spanning +-60 with a ragged tail, small enough for the full oracle
    q, k, v = make_qkv(1, 2, 777, 128, dtype, seed_base=555, dist="stress")
    scale = default_scale(128)
    o, lse = _run(iofa.forward, q, k, v, scale, dev)
    o_ref, lse_ref = oracle_full(q, k, v, scale)
    assert_parity(o, lse, o_ref, lse_ref, q.dtype, f"stress {dtype}")


def test_fused_many_heads(dev):
    # a grid of 4096 workgroups over short sequences; every head checked
    q, k, v = make_qkv(8, 256, 130, 64, "bf16", seed_base=77)
    scale = default_scale(64)
    o, lse = _run(iofa.forward, q, k, v, scale, dev)
    o_ref, lse_ref = oracle_full(q, k, v, scale)
    assert_parity(o, lse, o_ref, lse_ref, q.dtype, "many heads")


# Lengths for the 8-wave form: one to nine 32-key tiles, ragged tails, and
# the first length that takes two query tiles of 256 rows per head.
EIGHT_WAVE_N = [1, 17, 32, 33, 64, 65, 100, 129, 255, 256, 257]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fused_8wave_form_short_and_ragged(dtype, dev):
    # At d = 128 the launch takes workgroups of 8 waves (256 query rows) when
    # N fills at least one 4-wave tile (128 rows) and B*H*ceil(N/256) reaches
    # the CU count (256 on MI355X): 256 heads do so from N = 129 on, shorter
    # heads take 4-wave workgroups.  The last query tile leaves waves without
    # any query row (they only copy and synchronise) at every length here but
    # 100, 255 and 256: 3 of 4 at N <= 32, 7 of 8 at N = 257.  Every element of O
    # and LSE, NaN-filled before the launch, against the oracle.
    H = 256
    for N in EIGHT_WAVE_N:
        q, k, v = make_qkv(1, H, N, 128, dtype, seed_base=9000 + N)
        scale = default_scale(128)
        _say(f"fused 8-wave {dtype} H={H} N={N}")
        o, lse = nan_outputs(q, dev)
        iofa.fa_fwd(q.to(dev), k.to(dev), v.to(dev), o, lse, scale)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle_full(q, k, v, scale)
        assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, q.dtype, f"8-wave {dtype} N={N}")


@pytest.mark.parametrize("heads", [255, 256])
def test_fused_wave_form_boundary(heads, dev):
    # one query tile per head: 255 workgroups take the 4-wave form (255 * 2
    # workgroups of 128 rows), 256 the 8-wave form; both against the oracle
    q, k, v = make_qkv(1, heads, 200, 128, "bf16", seed_base=9500 + heads)
    scale = default_scale(128)
    _say(f"fused wave-form boundary H={heads}")
    o, lse = nan_outputs(q, dev)
    iofa.fa_fwd(q.to(dev), k.to(dev), v.to(dev), o, lse, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_full(q, k, v, scale)
    assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, q.dtype, f"boundary H={heads}")


@pytest.mark.parametrize("d", [64, 128])
def test_fused_long_heads_every_element(d, dev):
    # heads with more query tiles than an XCD runs at once (48 workgroups of
    # 256 rows at d = 128, 96 of 128 rows at d = 64, against 32 and 64 per
    # XCD), so each head takes more than one round; every element against
    # the oracle
    N = 12288
    q, k, v = make_qkv(1, 2, N, d, "bf16", seed_base=4242 + d)
    scale = default_scale(d)
    _say(f"fused long heads d={d} N={N}")
    o, lse = nan_outputs(q, dev)
    iofa.fa_fwd(q.to(dev), k.to(dev), v.to(dev), o, lse, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_full(q, k, v, scale)
    res = assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, q.dtype, f"long heads d={d}")
    _say(f"  max_abs={res[0]:.3e} rel_f={res[1]:.3e} lse={res[2]:.3e}")


def test_fused_other_scales(dev):
    q, k, v = make_qkv(1, 2, 300, 128, "bf16", seed_base=91)
    for scale in (0.0, -0.125, 0.5):
        o, lse = _run(iofa.forward, q, k, v, scale, dev)
        o_ref, lse_ref = oracle_full(q, k, v, scale)
        # scale 0.5 at d=128 makes rows nearly one-hot, so |O| reaches ~3.5
        assert_parity(o, lse, o_ref, lse_ref, q.dtype, f"scale={scale}",
                      output_rounding=True)


# ------------------------------------------------------ invariants on GPU

def test_shift_invariance_on_gpu(dev):
    # K and u on a 1/8 grid in [-4, 4], so K + 1 u^T is exact in bf16
    g = torch.Generator().manual_seed(2024)
    B, H, N, d = 1, 4, 2000, 128
    q = (torch.randint(-32, 33, (B, H, N, d), generator=g) / 8.0).to(torch.bfloat16)
    k = (torch.randint(-32, 33, (B, H, N, d), generator=g) / 8.0).to(torch.bfloat16)
    v = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16)
    u = torch.randint(-32, 33, (d,), generator=g) / 8.0
    k2 = (k.float() + u).to(torch.bfloat16)
    assert torch.equal(k2.float(), k.float() + u)
    scale = default_scale(d)
    o1, l1 = _run(iofa.forward, q, k, v, scale, dev)
    o2, l2 = _run(iofa.forward, q, k2, v, scale, dev)
    shift = np.float32(scale) * (widen(q) @ u.double().numpy())
    dl = l2.double().numpy() - l1.double().numpy()
    assert np.abs(dl - shift).max() <= 2e-3 * max(1.0, np.abs(shift).max())
    # two outputs rounded independently to bf16 may differ by one unit in the
    # last place of |O| (2u|O|, u = 2^-8) on top of the fused bar
    o1w, o2w = widen(o1), widen(o2)
    excess = np.abs(o2w - o1w) - 2.0 * 2.0 ** -8 * np.abs(o1w)
    rel_f = np.linalg.norm(o2w - o1w) / np.linalg.norm(o1w)
    assert excess.max() <= 1e-2 and rel_f <= 5e-3


def test_deterministic(dev):
    q, k, v, scale, _ = workload_qkv(2)
    o1, l1 = _run(iofa.forward, q, k, v, scale, dev)
    o2, l2 = _run(iofa.forward, q, k, v, scale, dev)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("dtype,N,d", [("bf16", 8191, 128), ("fp16", 129, 64), ("bf16", 77, 128),
                                         ("fp32", 100, 128)])
def test_no_writes_outside_outputs(dtype, N, d, dev):
    B, H = 1, 2
    q, k, v = (t.to(dev) for t in make_qkv(B, H, N, d, dtype, seed_base=5))
    guard = 4096
    n_o = B * H * N * d
    obuf = torch.full((guard + n_o + guard,), float("nan"), dtype=DT[dtype], device=dev)
    lbuf = torch.full((guard + B * H * N + guard,), -7.0, dtype=torch.float32, device=dev)
    o = obuf[guard:guard + n_o].view(B, H, N, d)
    lse = lbuf[guard:guard + B * H * N].view(B, H, N)
    iofa.fa_fwd(q, k, v, o, lse, default_scale(d))
    torch.cuda.synchronize()
    assert torch.isnan(obuf[:guard]).all() and torch.isnan(obuf[-guard:]).all()
    assert (lbuf[:guard] == -7.0).all() and (lbuf[-guard:] == -7.0).all()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_runs_on_caller_stream(dev):
    q, k, v = (t.to(dev) for t in make_qkv(1, 2, 512, 128, "bf16", seed_base=3))
    s = torch.cuda.Stream(device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(1, 2, 512, dtype=torch.float32, device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        iofa.fa_fwd(q, k, v, o, lse, default_scale(128), stream=s)
    s.synchronize()
    o_ref, lse_ref = oracle_full(q.cpu(), k.cpu(), v.cpu(), default_scale(128))
    assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, torch.bfloat16, "side stream")


def test_errors_surface_through_binding(dev):
    q, k, v = (t.to(dev) for t in make_qkv(1, 1, 64, 128, "bf16", seed_base=1))
    lse = torch.empty(1, 1, 64, dtype=torch.float32, device=dev)
    with pytest.raises(iofa.FaError) as ei:
        iofa.fa_fwd(q, k, v, q, lse, 0.1)          # O aliases Q
    assert ei.value.status == 7
    with pytest.raises(iofa.FaError) as ei:
        iofa.fa_fwd(q, k, v, torch.empty_like(q), lse, float("inf"))
    assert ei.value.status == 6
    q96 = torch.zeros(1, 1, 64, 96, dtype=torch.bfloat16, device=dev)
    with pytest.raises(iofa.FaError) as ei:
        iofa.fa_fwd(q96, q96.clone(), q96.clone(), q96.clone(), lse, 0.1)
    assert ei.value.status == 3


def test_host_tensors_are_rejected_before_the_library(dev):
    # a host pointer would reach the kernels as an unusable address: the
    # binding refuses it (output, statistics or workspace alike)
    q, k, v = (t.to(dev) for t in make_qkv(1, 1, 64, 128, "bf16", seed_base=2))
    o = torch.empty_like(q)
    lse = torch.empty(1, 1, 64, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError, match="on a GPU"):
        iofa.fa_fwd(q, k, v, o, torch.empty(1, 1, 64), 0.1)
    with pytest.raises(ValueError):
        iofa.fa_fwd(q, k, v, o.cpu(), lse, 0.1)
    ws = torch.empty(iofa.fa_splitkv_workspace_bytes(1, 1, 64, 128, q.dtype, 2), dtype=torch.uint8)
    with pytest.raises(ValueError, match="on a GPU"):
        iofa.fa_fwd_splitkv(q, k, v, o, lse, ws, 0.1, 2)
    x = torch.zeros(2, 100, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError, match="on a GPU"):
        iofa.fa_softmax_rows(x, torch.empty(2, 100, dtype=torch.bfloat16), None)
    torch.cuda.synchronize()


# ----------------------------------------------------------- naive path
#
# The naive path stores S and P in the input type, so its error is not held
# to the fused path's bar but to the per-element bound its own arithmetic
# gives (tests/helpers.py: naive_output_bound).  fp32 inputs keep S and P in
# fp32 and take the fused bar.

def check_naive(o, lse, q, k, v, scale, o_ref, lse_ref, label, rows=None):
    """Hold naive-path outputs (CPU tensors, the rows ``rows`` of every head
    or all rows) to the fp32 bar or to the derived 16-bit bound."""
    max_abs, rel_f, lse_err = errors(o, lse, o_ref, lse_ref)
    if q.dtype == torch.float32:
        assert_parity(o, lse, o_ref, lse_ref, q.dtype, label)
        _say(f"  {label}: max_abs={max_abs:.3e} rel_f={rel_f:.3e} lse={lse_err:.3e}")
        return
    bound, lbound = naive_output_bound(q, k, v, scale, o_ref, lse_ref, rows=rows)
    err = np.abs(widen(o) - o_ref)
    worst = float(np.max(err / bound)) if err.size else 0.0
    msg = (f"{label}: max_abs={max_abs:.3e} rel_f={rel_f:.3e} lse={lse_err:.3e} "
           f"worst err/bound={worst:.3f}")
    _say("  " + msg)
    assert np.isfinite(widen(o)).all(), msg
    assert (err <= bound).all(), msg
    if lse is not None:
        lerr = np.abs(lse.double().numpy() - lse_ref)
        assert (lerr <= lbound).all(), msg + f" lse worst err/bound={np.max(lerr / lbound):.3f}"


def _naive_prefilled(q, k, v, scale, dev):
    o, lse = nan_outputs(q, dev)
    B, H, N, _ = q.shape
    nbytes = max(iofa.fa_naive_workspace_bytes(B, H, N, q.dtype), 16)
    s_ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    p_ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    iofa.fa_naive_fwd(q.to(dev), k.to(dev), v.to(dev), o, lse, s_ws, p_ws, scale)
    torch.cuda.synchronize()
    del s_ws, p_ws
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("idx", [1, 2, 3, 5])
def test_naive_workload(idx, dev):
    # every element against the oracle
    q, k, v, scale, spec = workload_qkv(idx)
    _say(f"naive workload {idx}: {spec['name']}")
    o, lse = _naive_prefilled(q, k, v, scale, dev)
    o_ref, lse_ref = workload_oracle(idx)
    check_naive(o, lse, q, k, v, scale, o_ref, lse_ref, f"naive w{idx} (every element)")


def test_naive_long_sequence_every_query_tile(dev):
    # B1 H32 N16384 d128: S and P take 16 GiB each.  Two rows of every
    # 128-row query tile, different rows in every head, plus the first and
    # last rows, against the oracle on those rows
    q, k, v, scale, spec = workload_qkv(4)
    _say(f"naive workload 4: {spec['name']}")
    o, lse = _naive_prefilled(q, k, v, scale, dev)
    rows = tile_rows(spec["N"], spec["H"], seed=4)
    for h in range(spec["H"]):
        sl = slice(h, h + 1)
        o_ref, lse_ref = oracle_rows(q[:, sl], k[:, sl], v[:, sl], scale, rows[h])
        check_naive(o[:, sl, rows[h]], lse[:, sl, rows[h]], q[:, sl], k[:, sl], v[:, sl],
                    scale, o_ref, lse_ref, f"naive w4 head {h} ({rows.shape[1]} rows)",
                    rows=rows[h])


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_naive_ragged(dtype, dev):
    for N in (1, 7, 64, 65, 200, 1000):
        for d in (64, 128):
            q, k, v = make_qkv(1, 2, N, d, dtype, seed_base=3 * N + d)
            scale = default_scale(d)
            _say(f"naive ragged {dtype} d={d} N={N}")
            o, lse = _run(iofa.naive_forward, q, k, v, scale, dev)
            o_ref, lse_ref = oracle_full(q, k, v, scale)
            check_naive(o, lse, q, k, v, scale, o_ref, lse_ref, f"naive {dtype} d={d} N={N}")


def test_naive_without_lse(dev):
    q, k, v = make_qkv(1, 2, 300, 64, "bf16", seed_base=8)
    o, lse = _run(iofa.naive_forward, q, k, v, default_scale(64), dev, want_lse=False)
    assert lse is None
    o_ref, lse_ref = oracle_full(q, k, v, default_scale(64))
    check_naive(o, None, q, k, v, default_scale(64), o_ref, lse_ref, "naive without lse")


@pytest.mark.parametrize("dtype,N,d", [("bf16", 1000, 128), ("fp16", 65, 64), ("fp32", 100, 128)])
def test_naive_no_writes_outside_outputs(dtype, N, d, dev):
    # O, LSE and both workspaces sit inside guard regions that must come back
    # unchanged (the scores kernel drops pieces of S outside the valid rows
    # and keys through range-checked stores; the other kernels bound their
    # writes by index)
    B, H = 1, 2
    q, k, v = (t.to(dev) for t in make_qkv(B, H, N, d, dtype, seed_base=7 * N + d))
    guard = 4096
    nb = iofa.fa_naive_workspace_bytes(B, H, N, q.dtype)
    s_buf = torch.full((guard + nb + guard,), 0xA5, dtype=torch.uint8, device=dev)
    p_buf = torch.full((guard + nb + guard,), 0x5A, dtype=torch.uint8, device=dev)
    n = B * H * N * d
    o_buf = torch.full((guard + n + guard,), float("nan"), dtype=q.dtype, device=dev)
    l_buf = torch.full((guard + B * H * N + guard,), float("nan"), dtype=torch.float32, device=dev)
    o = o_buf[guard:guard + n].view(B, H, N, d)
    lse = l_buf[guard:guard + B * H * N].view(B, H, N)
    iofa.fa_naive_fwd(q, k, v, o, lse, s_buf[guard:guard + nb], p_buf[guard:guard + nb],
                      default_scale(d))
    torch.cuda.synchronize()
    for buf, fill in ((s_buf, 0xA5), (p_buf, 0x5A)):
        assert bool((buf[:guard] == fill).all()) and bool((buf[guard + nb:] == fill).all())
    for buf, size in ((o_buf, n), (l_buf, B * H * N)):
        assert bool(torch.isnan(buf[:guard]).all()) and bool(torch.isnan(buf[guard + size:]).all())
    o_ref, lse_ref = oracle_full(q.cpu(), k.cpu(), v.cpu(), default_scale(d))
    check_naive(o.cpu(), lse.cpu(), q.cpu(), k.cpu(), v.cpu(), default_scale(d), o_ref, lse_ref,
                f"naive guards {dtype} N={N} d={d}")


def test_inputs_may_share_one_buffer(dev):
    # self-attention on one tensor: Q, K and V are the same device buffer
    x, _, _ = make_qkv(1, 2, 333, 128, "bf16", seed_base=95)
    xd = x.to(dev)
    o = torch.empty_like(xd)
    lse = torch.empty((1, 2, 333), dtype=torch.float32, device=dev)
    iofa.fa_fwd(xd, xd, xd, o, lse, default_scale(128))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_full(x, x, x, default_scale(128))
    # q . q dominates each row (scores near |q|^2 / sqrt(d)), so |O| reaches |x|
    assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, x.dtype, "Q = K = V", output_rounding=True)
    dq, dk, dv = iofa.backward(xd, xd, xd, o, lse, torch.ones_like(xd))
    torch.cuda.synchronize()
    assert all(torch.isfinite(t).all() for t in (dq, dk, dv))
