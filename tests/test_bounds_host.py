"""CPU checks of the derived per-element bars used by the GPU parity tests:
a plain-torch model of the arithmetic each bar covers stays within it, and
a model with coarser arithmetic than the bar assumes does not.  The models
are test scaffolding, not a reference: parity itself is always against the
fp64 oracle."""

import numpy as np
import pytest
import torch

from helpers import naive_output_bound, oracle_full, tile_rows, widen
from workloads import default_scale, make_qkv


def _naive_model(q, k, v, scale, store):
    """S = scale q k^T in fp32, stored in ``store``; fp32 softmax; P stored
    in ``store``; O = P V in fp32, rounded to the input type."""
    s = (torch.matmul(q.float(), k.float().transpose(-1, -2)) * np.float32(scale)).to(store)
    s = s.float()
    m = s.amax(dim=-1, keepdim=True)
    f = torch.exp(s - m)
    l_ = f.sum(dim=-1, keepdim=True)
    p = (f / l_).to(store).float()
    o = torch.matmul(p, v.float()).to(q.dtype)
    return o, (m + torch.log(l_))[..., 0]


@pytest.mark.parametrize("dtype,dist,N", [("bf16", "normal", 300), ("fp16", "stress", 257),
                                          ("bf16", "stress", 200)])
def test_naive_bound_covers_its_model(dtype, dist, N):
    q, k, v = make_qkv(1, 2, N, 64, dtype, seed_base=31 + N, dist=dist)
    scale = default_scale(64)
    o_ref, lse_ref = oracle_full(q, k, v, scale)
    bound, lbound = naive_output_bound(q, k, v, scale, o_ref, lse_ref)
    o, lse = _naive_model(q, k, v, scale, q.dtype)
    err = np.abs(widen(o) - o_ref)
    assert (err <= bound).all(), float((err / bound).max())
    assert (np.abs(lse.double().numpy() - lse_ref) <= lbound).all()
    # not vacuous: the bar is within a small factor of the model's worst error
    assert float((err / bound).max()) > 0.05


def test_naive_bound_rejects_coarser_storage():
    # scores and weights stored in E4M3 (3 mantissa bits) instead of bf16 (7)
    q, k, v = make_qkv(1, 2, 300, 64, "bf16", seed_base=5)
    scale = default_scale(64)
    o_ref, lse_ref = oracle_full(q, k, v, scale)
    bound, _ = naive_output_bound(q, k, v, scale, o_ref, lse_ref)
    o, _ = _naive_model(q, k, v, scale, torch.float8_e4m3fn)
    assert (np.abs(widen(o) - o_ref) > bound).any()


def test_tile_rows_cover_every_tile_of_every_head():
    N, H = 16384, 32
    rows = tile_rows(N, H, seed=4)
    assert rows.shape[0] == H and rows.min() == 0 and (rows[:, -1] == N - 1).all()
    for h in range(H):
        tiles = set((rows[h] // 128).tolist())
        assert tiles == set(range(N // 128))
    # heads get different rows
    assert len({tuple(r) for r in rows.tolist()}) == H
