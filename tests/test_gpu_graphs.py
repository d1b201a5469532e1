"""The C-ABI entry points inside HIP graphs: each call is captured once into
a graph (torch.cuda.CUDAGraph, on torch's capture stream, which the binding
passes as the call's stream) and replayed several times, with the program's
own eager work and a synchronisation between replays; every replay must
reproduce the eager result bit for bit (all the kernels are deterministic,
allocate nothing and issue no memsets)."""

import pytest
import torch

import io_aware_softmax_04_amd as iofa
from workloads import default_scale, make_qkv, make_qkv_fp8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    iofa.load_library()
    return torch.device("cuda:0")


def _replays_match(call, outputs, dev, replays=3):
    """Run call() eagerly, capture it, replay; compare every replay's outputs
    with the eager ones."""
    call()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outputs]
    for t in outputs:
        t.fill_(0)                     # replays must rewrite every element
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):      # warm-up on a side stream, as graph capture expects
        call()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    noise = torch.randn(1 << 20, device=dev)
    for r in range(replays):
        for t in outputs:
            t.fill_(0)
        noise.mul_(1.0001).add_(0.5)   # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(outputs, eager):
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), f"replay {r}"


def test_fused_forward_in_a_graph(dev):
    q, k, v = (t.to(dev) for t in make_qkv(1, 4, 1000, 128, "bf16", seed_base=31))
    o = torch.empty_like(q)
    lse = torch.empty((1, 4, 1000), dtype=torch.float32, device=dev)
    _replays_match(lambda: iofa.fa_fwd(q, k, v, o, lse, default_scale(128)), [o, lse], dev)


def test_splitkv_forward_in_a_graph(dev):
    q, k, v = (t.to(dev) for t in make_qkv(1, 2, 2000, 64, "fp16", seed_base=32))
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, 2000), dtype=torch.float32, device=dev)
    g = 5
    ws = torch.empty(iofa.fa_splitkv_workspace_bytes(1, 2, 2000, 64, q.dtype, g),
                     dtype=torch.uint8, device=dev)
    _replays_match(lambda: iofa.fa_fwd_splitkv(q, k, v, o, lse, ws, default_scale(64), g),
                   [o, lse], dev)


@pytest.mark.parametrize("Nq,Nk", [(1, 3000), (130, 700)])
def test_splitkv_qk_forward_in_a_graph(Nq, Nk, dev):
    # queries and keys of different lengths: one decode row, and a query
    # block longer than the key sequence
    q, _, _ = make_qkv(1, 3, Nq, 128, "bf16", seed_base=36)
    _, k, v = make_qkv(1, 3, Nk, 128, "bf16", seed_base=37)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((1, 3, Nq), dtype=torch.float32, device=dev)
    g = iofa.fa_splitkv_qk_num_splits(1, 3, Nq, Nk, 128, q.dtype)
    nbytes = iofa.fa_splitkv_qk_workspace_bytes(1, 3, Nq, Nk, 128, q.dtype, g)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    _replays_match(lambda: iofa.fa_fwd_splitkv_qk(q, k, v, o, lse, ws, default_scale(128), g),
                   [o, lse], dev)


def test_backward_in_a_graph(dev):
    q, k, v = (t.to(dev) for t in make_qkv(1, 2, 700, 128, "bf16", seed_base=33))
    do = torch.randn_like(q)
    o, lse = iofa.forward(q, k, v)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(iofa.fa_bwd_workspace_bytes(1, 2, 700), dtype=torch.uint8, device=dev)
    _replays_match(lambda: iofa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, default_scale(128)),
                   [dq, dk, dv], dev)


def test_fp8_forward_in_a_graph(dev):
    (q8, k8, v8), (sq, sk, sv) = make_qkv_fp8(1, 2, 900, 128, seed_base=34)
    q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, 2, 900), dtype=torch.float32, device=dev)
    _replays_match(lambda: iofa.fa_fwd_fp8(q8, k8, v8, o, lse, default_scale(128), sq, sk, sv),
                   [o, lse], dev)


@pytest.mark.parametrize("n", [3000, 50000, 20001, 1 << 20])
def test_row_softmax_in_a_graph(n, dev):
    # one chunk; 4 slices held in registers (one pass, with its clear and
    # repair kernels); scalar two passes; 16-byte two passes (64 slices)
    g = torch.Generator().manual_seed(n)
    x = (torch.randn((4, n), generator=g) * 3).to(torch.bfloat16).to(dev)
    y = torch.empty_like(x)
    lse = torch.empty(4, dtype=torch.float32, device=dev)
    nb = iofa.fa_softmax_workspace_bytes(4, n, x.dtype)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    _replays_match(lambda: iofa.fa_softmax_rows(x, y, lse, ws if nb else None), [y, lse], dev)


def test_naive_forward_in_a_graph(dev):
    q, k, v = (t.to(dev) for t in make_qkv(1, 2, 300, 64, "bf16", seed_base=35))
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, 300), dtype=torch.float32, device=dev)
    nb = iofa.fa_naive_workspace_bytes(1, 2, 300, q.dtype)
    s_ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    p_ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    _replays_match(lambda: iofa.fa_naive_fwd(q, k, v, o, lse, s_ws, p_ws, default_scale(64)),
                   [o, lse], dev)


def test_graph_replay_reads_the_current_inputs(dev):
    # a captured call reads its inputs when replayed: after the inputs are
    # overwritten in place, a replay gives the eager result on the new values
    q, k, v = (t.to(dev) for t in make_qkv(1, 2, 777, 128, "bf16", seed_base=36))
    q2, k2, v2 = (t.to(dev) for t in make_qkv(1, 2, 777, 128, "bf16", seed_base=37))
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, 777), dtype=torch.float32, device=dev)
    call = lambda: iofa.fa_fwd(q, k, v, o, lse, default_scale(128))  # noqa: E731
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    o_ref, lse_ref = iofa.forward(q2, k2, v2)
    for dst, src in ((q, q2), (k, k2), (v, v2)):
        dst.copy_(src)
    o.fill_(0)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.uint8), o_ref.view(torch.uint8))
    assert torch.equal(lse, lse_ref)
