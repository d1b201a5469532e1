"""GPU parity of the split-KV forward and of the merge entry point against
the fp64 oracle (partial attention over key ranges, and the block merge),
called through the C ABI."""

import numpy as np
import pytest
import torch

import io_aware_softmax_04_amd as iofa
import oracle
from helpers import (TOL, assert_parity, errors, nan_outputs, oracle_full, oracle_rows,
                     sample_rows, widen)
from workloads import default_scale, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    iofa.load_library()
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _key_tile(dtype, d):
    return 32 if (dtype == "fp32" or d == 128) else 64


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_splitkv_matches_oracle(dtype, d, dev):
    for N, splits in ((65, 2), (200, 3), (1000, 0), (1025, 5), (777, 64), (300, 1)):
        q, k, v = make_qkv(1, 2, N, d, dtype, seed_base=31 * N + d)
        scale = default_scale(d)
        g = iofa.fa_splitkv_num_splits(1, 2, N, d, q.dtype, splits)
        _say(f"splitkv {dtype} d={d} N={N} requested={splits} G={g}")
        o, lse = iofa.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), scale, splits)
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle_full(q, k, v, scale)
        assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, q.dtype,
                      f"splitkv {dtype} d={d} N={N} G={g}")


def test_splitkv_one_gpu_share_of_the_headline_workload(dev):
    # B=2 H=2 N=4096 d=128: the per-GPU share of the B=2 H=16 workload split
    # by heads over 8 GPUs; 128 query-tile workgroups, so 4 key ranges
    q, k, v = make_qkv(2, 2, 4096, 128, "bf16", seed_base=3000)
    scale = default_scale(128)
    assert iofa.fa_splitkv_num_splits(2, 2, 4096, 128, q.dtype, 0) == 4
    o, lse = iofa.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_full(q, k, v, scale)
    res = assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, q.dtype,
                        "splitkv B2 H2 N4096 (every element)")
    _say(f"  max_abs={res[0]:.3e} rel_f={res[1]:.3e} lse={res[2]:.3e}")


def test_splitkv_stress_distribution(dev):
    q, k, v = make_qkv(1, 2, 2000, 128, "fp16", seed_base=5555, dist="stress")
    scale = default_scale(128)
    o, lse = iofa.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), scale, 5)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_full(q, k, v, scale)
    assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, q.dtype, "splitkv stress G=5")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64), ("fp32", 128)])
def test_splitkv_partials_match_partial_attention(dtype, d, dev):
    # the partial pass on its own: the workspace holds, per key range, the
    # attention over that range's keys (oracle.partial_attention)
    B, H, N, G = 1, 2, 700, 3
    q, k, v = make_qkv(B, H, N, d, dtype, seed_base=77 + d)
    scale = default_scale(d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(qd)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=dev)
    nbytes = iofa.fa_splitkv_workspace_bytes(B, H, N, d, q.dtype, G)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    iofa.fa_fwd_splitkv(qd, kd, vd, o, lse, ws, scale, G)
    torch.cuda.synchronize()
    flat = ws.view(torch.float32).cpu()
    o_part = flat[:G * B * H * N * d].view(G, B, H, N, d).double().numpy()
    lse_part = flat[G * B * H * N * d:].view(G, B, H, N).double().numpy()
    bc = _key_tile(dtype, d)
    nt = (N + bc - 1) // bc
    tol = TOL[q.dtype]
    for s in range(G):
        k0, k1 = s * nt // G * bc, min(N, (s + 1) * nt // G * bc)
        po, pl = oracle.partial_attention(widen(q), widen(k), widen(v),
                                          float(np.float32(scale)), k0, k1)
        d_o = np.abs(o_part[s] - po)
        assert d_o.max() <= tol["o_abs"], (s, d_o.max())
        assert np.linalg.norm(o_part[s] - po) / np.linalg.norm(po) <= tol["o_relf"]
        assert np.abs(lse_part[s] - pl).max() <= tol["lse_abs"], s
    o_ref, lse_ref = oracle_full(q, k, v, scale)
    assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, q.dtype, f"splitkv {dtype} d={d} G=3")


# Queries and keys of different lengths: q (B, H, Nq, d) against k, v
# (B, H, Nk, d).  The oracle is the attention definition over all Nk keys
# (oracle.partial_attention over the whole key range).  Decode (Nq = 1) with
# short, ragged and long key sequences, and one sequence over another, both
# shorter and longer.
QK_SHAPES = [(1, 1), (1, 33), (1, 1000), (1, 4097), (3, 700), (300, 1000), (1000, 77), (129, 4096)]


def _qk_inputs(B, H, Nq, Nk, d, dtype, seed):
    q, _, _ = make_qkv(B, H, Nq, d, dtype, seed_base=seed)
    _, k, v = make_qkv(B, H, Nk, d, dtype, seed_base=seed + 7919)
    return q, k, v


def _run_qk(q, k, v, scale, splits, dev):
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = nan_outputs(q, dev)
    nbytes = iofa.fa_splitkv_qk_workspace_bytes(B, H, Nq, Nk, d, q.dtype, splits)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev) if nbytes else None
    iofa.fa_fwd_splitkv_qk(qd, kd, vd, o, lse, ws, scale, splits)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_splitkv_qk_matches_oracle(dtype, d, dev):
    B, H = 2, 3
    scale = default_scale(d)
    for Nq, Nk in QK_SHAPES:
        q, k, v = _qk_inputs(B, H, Nq, Nk, d, dtype, 101 * Nq + Nk + d)
        po, pl = oracle.partial_attention(widen(q), widen(k), widen(v),
                                          float(np.float32(scale)), 0, Nk)
        for splits in (0, 1, 3):
            g = iofa.fa_splitkv_qk_num_splits(B, H, Nq, Nk, d, q.dtype, splits)
            _say(f"splitkv qk {dtype} d={d} Nq={Nq} Nk={Nk} requested={splits} G={g}")
            o, lse = _run_qk(q, k, v, scale, splits, dev)
            assert_parity(o, lse, po, pl, q.dtype, f"qk {dtype} d={d} Nq={Nq} Nk={Nk} G={g}")


def test_splitkv_qk_decode_at_the_benchmarked_size(dev):
    # one query row per head against the 4096 keys of B2 H16 d128: every
    # element of O and LSE against the oracle
    B, H, Nq, Nk, d = 2, 16, 1, 4096, 128
    q, k, v = _qk_inputs(B, H, Nq, Nk, d, "bf16", 6060)
    scale = default_scale(d)
    g = iofa.fa_splitkv_qk_num_splits(B, H, Nq, Nk, d, q.dtype, 0)
    assert g == 8
    o, lse = _run_qk(q, k, v, scale, 0, dev)
    po, pl = oracle.partial_attention(widen(q), widen(k), widen(v), float(np.float32(scale)), 0, Nk)
    res = assert_parity(o, lse, po, pl, q.dtype, "decode B2 H16 Nk4096 G=8")
    _say(f"  max_abs={res[0]:.3e} rel_f={res[1]:.3e} lse={res[2]:.3e}")


def test_splitkv_qk_with_equal_lengths_is_splitkv(dev):
    # Nq = Nk: the same launches as fa_fwd_splitkv, so the same bits
    q, k, v = make_qkv(1, 2, 1000, 128, "bf16", seed_base=808)
    scale = default_scale(128)
    for splits in (0, 1, 4):
        o1, l1 = _run_qk(q, k, v, scale, splits, dev)
        o2, l2 = iofa.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), scale, splits)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.cpu().view(torch.int16))
        assert torch.equal(l1, l2.cpu())


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("d", [64, 128])
def test_merge_entry_point(out_dtype, d, dev):
    rng = np.random.default_rng(d)
    # G covers every load-group size of the kernel (1, 2, 4, 8 and 16 with
    # several groups and LSE chunks)
    for G, rows in ((1, 5), (2, 333), (3, 64), (4, 100), (7, 1000), (9, 77), (33, 40),
                    (100, 20)):
        o_part = rng.standard_normal((G, rows, d)).astype(np.float32)
        lse_part = rng.uniform(-20, 20, (G, rows)).astype(np.float32)
        if G > 1:
            lse_part[0, ::3] = -np.inf            # blocks without keys
            lse_part[:, 1::7] = -np.inf           # rows whose blocks are all empty
        o_ref, lse_ref = oracle.merge_partials(o_part.astype(np.float64),
                                               lse_part.astype(np.float64))
        o = torch.empty(rows, d, dtype=out_dtype, device=dev)
        lse = torch.empty(rows, dtype=torch.float32, device=dev)
        iofa.fa_merge_partials(torch.from_numpy(o_part).to(dev),
                               torch.from_numpy(lse_part).to(dev), o, lse)
        torch.cuda.synchronize()
        got = widen(o.cpu())
        u = {torch.float32: 2.0 ** -24, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}
        # output rounding u|O| plus fp32 arithmetic over G terms
        bound = u[out_dtype] * np.abs(o_ref) + 1e-5 * (1 + np.abs(o_ref))
        assert np.all(np.abs(got - o_ref) <= bound), (G, rows, np.abs(got - o_ref).max())
        got_lse = lse.cpu().double().numpy()
        empty = np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(got_lse), empty)
        assert np.all(got[empty] == 0)
        fin = ~empty
        assert np.abs(got_lse[fin] - lse_ref[fin]).max() <= 1e-5 * (1 + np.abs(lse_ref[fin]).max())


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64)])
def test_key_blocking_does_not_change_the_result(dtype, d, dev):
    # Any division of the keys into blocks gives the same exact attention (the
    # online recurrence adds blocks one at a time, [xinc] "7. Online Softmax",
    # and [jiahao] "增量求解 softmax" merges any two).  The split-KV forward cuts
    # the key tiles into G ranges and merges them, so every G is a different
    # blocking and summation order: each meets the parity bar against the
    # oracle and against the fused kernel's result; G = 1 runs the fused kernel.
    N = 1000                                      # ragged: not a multiple of 32 or 64
    q, k, v = make_qkv(1, 4, N, d, dtype, seed_base=4242 + d)
    scale = default_scale(d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o_f, lse_f = iofa.forward(qd, kd, vd, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_full(q, k, v, scale)
    assert_parity(o_f.cpu(), lse_f.cpu(), o_ref, lse_ref, q.dtype, f"fused {dtype} d={d}")
    tol = TOL[q.dtype]
    for g in (1, 2, 3, 5, 8):
        assert iofa.fa_splitkv_num_splits(1, 4, N, d, q.dtype, g) == g
        _say(f"blocking {dtype} d={d} N={N} G={g}")
        o, lse = iofa.forward_splitkv(qd, kd, vd, scale, g)
        torch.cuda.synchronize()
        if g == 1:
            assert torch.equal(o, o_f) and torch.equal(lse, lse_f)
            continue
        assert_parity(o.cpu(), lse.cpu(), o_ref, lse_ref, q.dtype, f"splitkv G={g}")
        diff = (o.float() - o_f.float()).abs()
        assert diff.max().item() <= tol["o_abs"], (g, diff.max().item())
        rel = (torch.linalg.norm(o.float() - o_f.float()) / torch.linalg.norm(o_f.float())).item()
        assert rel <= tol["o_relf"], (g, rel)
        assert (lse - lse_f).abs().max().item() <= tol["lse_abs"], g
