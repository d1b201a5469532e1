"""GPU parity at the size limits of the C ABI: the longest sequence a head
may have at d = 128 (N * d < 2^31 allows N up to 2^24 - 1; N = 2^20 here, a
head of 2^27 elements, 256 MiB of bf16 per tensor), and the longest rows of
the standalone softmax that these tests run (2^27 elements).  These runs use
the large element offsets, range-checked buffer lengths and grid sizes that
the smaller tests do not reach.  Outputs are checked on sampled query rows
(first, last and seeded random rows) against the fp64 oracle, with the same
bars as the other parity tests."""

import numpy as np
import pytest
import torch

import io_aware_softmax_04_amd as iofa
import oracle
from helpers import assert_parity, check_backward, fp8_output_bound, oracle_rows, sample_rows, widen
from workloads import default_scale, make_qkv, make_qkv_fp8

pytestmark = pytest.mark.gpu

N_LONG = 1 << 20


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    iofa.load_library()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def long_bf16():
    return make_qkv(1, 1, N_LONG, 128, "bf16", seed_base=777)


def test_fused_longest_sequence(long_bf16, dev):
    q, k, v = long_bf16
    o, lse = iofa.forward(q.to(dev), k.to(dev), v.to(dev))
    torch.cuda.synchronize()
    rows = sample_rows(N_LONG, seed=1, edge=8, middle=16)
    o_ref, lse_ref = oracle_rows(q, k, v, default_scale(128), rows)
    print(f"fused bf16 N=2^20: rows {rows.size}", flush=True)
    assert_parity(o[:, :, rows].cpu(), lse[:, :, rows].cpu(), o_ref, lse_ref, torch.bfloat16,
                  "fused N=2^20")


def test_splitkv_longest_sequence_one_head(long_bf16, dev):
    # one head: 8192 query tiles, split over the maximum number of key ranges
    q, k, v = long_bf16
    g = iofa.fa_splitkv_num_splits(1, 1, N_LONG, 128, torch.bfloat16, 64)
    assert g == 64
    o, lse = iofa.forward_splitkv(q.to(dev), k.to(dev), v.to(dev), num_splits=g)
    torch.cuda.synchronize()
    rows = sample_rows(N_LONG, seed=2, edge=8, middle=16)
    o_ref, lse_ref = oracle_rows(q, k, v, default_scale(128), rows)
    assert_parity(o[:, :, rows].cpu(), lse[:, :, rows].cpu(), o_ref, lse_ref, torch.bfloat16,
                  "split-KV N=2^20 G=64")


def test_fp8_longest_sequence(dev):
    (q8, k8, v8), (sq, sk, sv) = make_qkv_fp8(1, 1, N_LONG, 128, seed_base=778)
    scale = default_scale(128)
    o, lse = iofa.forward_fp8(q8.to(dev), k8.to(dev), v8.to(dev), sq, sk, sv)
    torch.cuda.synchronize()
    rows = sample_rows(N_LONG, seed=3, edge=8, middle=16)
    o_ref, lse_ref = oracle.fp8_attention_rows(q8.numpy(), k8.numpy(), v8.numpy(), scale,
                                               sq, sk, sv, rows)
    bound, eps = fp8_output_bound(q8, k8, v8, scale, sq, sk, sv, o_ref, rows=rows)
    err = np.abs(widen(o[:, :, rows].cpu()) - o_ref)
    print(f"fp8 N=2^20: worst err/bar={np.max(err / bound):.3f}", flush=True)
    assert (err <= bound).all()
    lerr = np.abs(lse[:, :, rows].cpu().double().numpy() - lse_ref)
    assert (lerr <= eps + 1e-5 * (1 + np.abs(lse_ref))).all()


def test_backward_at_the_benchmark_head_shape(dev):
    # two heads of the benchmarked shape (N = 4096, d = 128), full gradients
    check_backward(1, 2, 4096, 128, "bf16", seed=4096, dev=dev, label="bf16 H2 N4096")


def test_backward_at_the_benchmark_workload(dev):
    # the whole benchmarked workload (B = 2, H = 16, N = 4096, d = 128: the
    # grid the bench times, 1024 workgroups per kernel), every gradient
    # against the fp64 oracle (about 20 s of host time)
    check_backward(2, 16, 4096, 128, "bf16", seed=3000, dev=dev, label="bf16 B2 H16 N4096")


def test_backward_at_the_numerics_stress_workload(dev):
    # the numerics-stress workload at full size (B = 2, H = 8, N = 8191, not a
    # tile multiple, fp16, scores spanning about +-60), every gradient against
    # the fp64 oracle (about 30 s of host time)
    check_backward(2, 8, 8191, 128, "fp16", seed=5000, dev=dev, dist="stress",
                   label="stress fp16 B2 H8 N8191")


def test_softmax_longest_rows(dev):
    g = torch.Generator().manual_seed(5)
    x = (torch.randn((2, 1 << 27), generator=g) * 4).to(torch.bfloat16)
    y, lse = iofa.softmax(x.to(dev), want_lse=True)
    torch.cuda.synchronize()
    y_ref, lse_ref = oracle.softmax_rows(widen(x))
    u = 2.0 ** -8
    excess = np.abs(widen(y.cpu()) - y_ref) - (u + 2e-5) * np.abs(y_ref) - 2.0 ** -134
    print(f"softmax 2 x 2^27: worst excess {excess.max():.3e}", flush=True)
    assert excess.max() <= 0
    assert np.all(np.abs(lse.cpu().double().numpy() - lse_ref) <= 2e-5 * (1 + np.abs(lse_ref)))
