"""The entry point that allocates nothing, fa_fwd_splitkv_noalloc, called
through the C ABI: its output against fa_fwd_splitkv's (the same split with
a caller-owned workspace) on two calls in a row, the second on a smaller
input, and against the oracle at the parity bar."""

import numpy as np
import pytest
import torch

import io_aware_softmax_04_amd as iofa
from helpers import assert_parity, nan_outputs, oracle_full
from workloads import default_scale, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    iofa.load_library()
    return torch.device("cuda:0")


def test_noalloc_matches_the_workspace_entry_point(dev):
    # the second call is smaller, so it reads only the part of the shared
    # scratch array it wrote itself
    cases = [(2, 2, 4096, 128, "bf16", 0, 1), (1, 3, 1500, 64, "fp16", 3, 2)]
    for B, H, N, d, dt, req, seed in cases:
        q, k, v = make_qkv(B, H, N, d, dt, seed_base=900 + seed)
        scale = default_scale(d)
        g = iofa.fa_splitkv_num_splits(B, H, N, d, q.dtype, req)
        need = iofa.fa_splitkv_workspace_bytes(B, H, N, d, q.dtype, req)
        print(f"noalloc {dt} B{B} H{H} N{N} d{d}: G={g}, partials {need} bytes", flush=True)
        assert g > 1 and 0 < need <= iofa.FA_NOALLOC_SCRATCH_BYTES
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        o1, l1 = nan_outputs(q, dev)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        iofa.fa_fwd_splitkv(qd, kd, vd, o1, l1, ws, scale, req)
        o2, l2 = nan_outputs(q, dev)
        iofa.fa_fwd_splitkv_noalloc(qd, kd, vd, o2, l2, scale, req)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)
        o_ref, lse_ref = oracle_full(q, k, v, scale)
        assert_parity(o2.cpu(), l2.cpu(), o_ref, lse_ref, q.dtype, f"noalloc {dt} N={N}")


def test_noalloc_refuses_a_split_beyond_the_scratch(dev):
    q, k, v = (t.to(dev) for t in make_qkv(8, 16, 1024, 128, "bf16", seed_base=5))
    need = iofa.fa_splitkv_workspace_bytes(8, 16, 1024, 128, q.dtype, 8)
    assert need > iofa.FA_NOALLOC_SCRATCH_BYTES
    o, lse = nan_outputs(q.cpu(), dev)
    with pytest.raises(iofa.FaError) as ei:
        iofa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, default_scale(128), 8)
    assert ei.value.status == 2 and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.isnan(o).all()          # nothing was enqueued
    # one split needs no scratch: the fused kernel, the same as fa_fwd
    iofa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, default_scale(128), 1)
    o_f, l_f = iofa.forward(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_f.view(torch.int16)) and torch.equal(lse, l_f)
    assert np.isfinite(lse.cpu().numpy()).all()
