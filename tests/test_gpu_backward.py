"""GPU parity of the backward pass (fa_bwd) against the fp64 gradient
oracle, through the C ABI.

The GPU side takes O and LSE from its own fused forward (check_backward in
helpers.py runs both and applies the bars below).  Error budget per
gradient element, relative to the gradient's scale: P and dS are rounded to
the input type for the products (u each, u = 2^-8 bf16, 2^-11 fp16), D is
formed from the rounded O (about u), and the output is rounded (u); the
terms of each sum carry independent rounding errors, so the relative
Frobenius error is a small multiple of u.  Bars: relative Frobenius 3u and
max-abs 12u times the largest reference magnitude of that gradient.

A gradient whose exact value is zero (dQ and dK with a single key, where
P = 1 and dS = dP - D = 0) is held to the fp32 summation-order difference
of dP and D over d terms instead: 4 d 2^-24 max|dO| max|V| times the factor
that turns dS into it (scale max|K| for dQ, scale max|Q| for dK)."""

import pytest
import torch

import io_aware_softmax_04_amd as iofa
from helpers import check_backward
from workloads import make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    iofa.load_library()
    return torch.device("cuda:0")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_matches_oracle(dtype, d, dev):
    for N in (1, 31, 32, 33, 100, 129, 300):
        check_backward(1, 2, N, d, dtype, seed=N * 13 + d, dev=dev, label=f"{dtype} d={d} N={N}")


def test_backward_larger_and_multi_head(dev):
    check_backward(2, 3, 1000, 128, "bf16", seed=1, dev=dev, label="bf16 B2 H3 N1000")


@pytest.mark.parametrize("dtype,d", [("fp16", 128), ("bf16", 128), ("bf16", 64)])
def test_backward_stress_distribution(dtype, d, dev):
    check_backward(1, 2, 500, d, dtype, seed=2 + d, dev=dev, dist="stress",
                   label=f"stress {dtype} d={d}")


def test_backward_is_deterministic(dev):
    q, k, v = (t.to(dev) for t in make_qkv(1, 4, 700, 128, "bf16", seed_base=3))
    do = torch.randn_like(q)
    o, lse = iofa.forward(q, k, v)
    a = iofa.backward(q, k, v, o, lse, do)
    b = iofa.backward(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_backward_no_writes_outside_gradients(dev):
    B, H, N, d = 1, 2, 300, 128
    q, k, v = (t.to(dev) for t in make_qkv(B, H, N, d, "bf16", seed_base=8))
    do = torch.randn_like(q)
    o, lse = iofa.forward(q, k, v)
    guard, n = 4096, B * H * N * d
    bufs = [torch.full((guard + n + guard,), float("nan"), dtype=torch.bfloat16, device=dev)
            for _ in range(3)]
    dq, dk, dv = (b[guard:guard + n].view(B, H, N, d) for b in bufs)
    ws = torch.empty(iofa.fa_bwd_workspace_bytes(B, H, N), dtype=torch.uint8, device=dev)
    iofa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, iofa.default_scale(d))
    torch.cuda.synchronize()
    for b in bufs:
        assert torch.isnan(b[:guard]).all() and torch.isnan(b[-guard:]).all()
    for g in (dq, dk, dv):
        assert torch.isfinite(g).all()
