"""Shared test helpers: running the oracle on the exact inputs the GPU sees,
tolerances, and comparisons."""

import numpy as np
import torch

import io_aware_softmax_04_amd as iofa
import oracle
from workloads import default_scale, make_qkv, raw_bits

# Parity bars.  16-bit inputs: max-abs 1e-2 and relative Frobenius 5e-3 on O
# (oracle fed the same rounded inputs); fp32 inputs: 1e-5 for both.  LSE:
# 1e-3 absolute for 16-bit inputs, 1e-5 for fp32.
TOL = {
    torch.float32: dict(o_abs=1e-5, o_relf=1e-5, lse_abs=1e-5),
    torch.float16: dict(o_abs=1e-2, o_relf=5e-3, lse_abs=1e-3),
    torch.bfloat16: dict(o_abs=1e-2, o_relf=5e-3, lse_abs=1e-3),
}


def widen(t):
    """Exact fp64 values of a CPU tensor, decoded by the oracle from its bits."""
    bits = raw_bits(t)
    if t.dtype == torch.bfloat16:
        return oracle.decode_bf16(bits)
    if t.dtype == torch.float16:
        return oracle.decode_f16(bits)
    return oracle.decode_f32(bits)


def oracle_full(q, k, v, scale):
    return oracle.standard_attention(widen(q), widen(k), widen(v), float(np.float32(scale)))


def oracle_rows(q, k, v, scale, rows):
    return oracle.standard_attention_rows(widen(q), widen(k), widen(v),
                                          float(np.float32(scale)), rows)


def errors(o_gpu, lse_gpu, o_ref, lse_ref):
    """(max-abs O, relative Frobenius O, max-abs LSE) of GPU outputs (CPU
    tensors, any dtype) against fp64 references."""
    o = widen(o_gpu.cpu()) if o_gpu.dtype != torch.float64 else o_gpu.numpy()
    d = o - o_ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    ref_norm = float(np.linalg.norm(o_ref))
    rel_f = float(np.linalg.norm(d) / ref_norm) if ref_norm > 0 else float(np.linalg.norm(d))
    lse_err = 0.0
    if lse_gpu is not None and lse_ref is not None and lse_ref.size:
        lse_err = float(np.abs(lse_gpu.cpu().double().numpy() - lse_ref).max())
    return max_abs, rel_f, lse_err


# Unit roundoff of the output type: rounding O itself moves it by up to
# u * |O|, which alone exceeds 1e-2 once |O| > 2.56 in bf16.
UNIT_ROUNDOFF = {torch.float32: 2.0 ** -24, torch.float16: 2.0 ** -11,
                 torch.bfloat16: 2.0 ** -8}


def assert_parity(o_gpu, lse_gpu, o_ref, lse_ref, dtype, label="", tol=None,
                  output_rounding=False):
    """Check the parity bar.  With ``output_rounding`` the max-abs bar is
    applied to |o - o_ref| - u * |o_ref| (u the output type's unit roundoff),
    for inputs whose outputs are large enough that rounding O to its own type
    exceeds the absolute bar."""
    t = dict(TOL[dtype]) if tol is None else tol
    max_abs, rel_f, lse_err = errors(o_gpu, lse_gpu, o_ref, lse_ref)
    if output_rounding:
        d = np.abs(widen(o_gpu.cpu()) - o_ref) - UNIT_ROUNDOFF[dtype] * np.abs(o_ref)
        max_abs = float(d.max()) if d.size else 0.0
    msg = (f"{label}: max_abs={max_abs:.3e} (<= {t['o_abs']:.0e}) rel_f={rel_f:.3e} "
           f"(<= {t['o_relf']:.0e}) lse={lse_err:.3e} (<= {t['lse_abs']:.0e})")
    assert np.isfinite(max_abs) and max_abs <= t["o_abs"], msg
    assert rel_f <= t["o_relf"], msg
    assert lse_err <= t["lse_abs"], msg
    return max_abs, rel_f, lse_err


def sample_rows(N, seed=0, edge=64, middle=64):
    """Query rows checked at full size: the first and last ``edge`` rows (the
    first and the ragged last tiles) plus ``middle`` seeded random rows."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(edge, N))) | set(range(max(0, N - edge), N))
    rows |= set(rng.integers(0, N, size=middle).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def fp8_output_bound(q8, k8, v8, scale, sq, sk, sv, o_ref, rows=None):
    """Per-element bar on O and per-row score-error bound eps of the FP8
    forward (derivation in tests/test_gpu_fp8.py's docstring), for the rows
    ``rows`` of every head, or all rows.  q8, k8, v8: CPU uint8 code
    tensors; o_ref: the oracle's output for those rows."""
    qd, kd, vd = (oracle.decode_e4m3(t.numpy()) for t in (q8, k8, v8))
    qv, kv, vv = oracle.fp8_values(q8.numpy(), k8.numpy(), v8.numpy(), sq, sk, sv)
    if rows is not None:
        qd, qv = qd[:, :, rows], qv[:, :, rows]
    c = abs(float(np.float32(scale))) * float(np.float32(sq)) * float(np.float32(sk))
    B, H = qd.shape[:2]
    bound = np.empty_like(o_ref)
    eps_all = np.empty(o_ref.shape[:3])
    for b in range(B):
        for h in range(H):
            mag = np.abs(qd[b, h]) @ np.abs(kd[b, h]).T            # sum_c |q8 k8|
            s = float(np.float32(scale)) * (qv[b, h] @ kv[b, h].T)
            eps = 2.0 ** -10 * c * mag.max(axis=1) + 2.0 ** -20 * (1 + np.abs(s).max(axis=1))
            w = np.exp(s - s.max(axis=1, keepdims=True))
            r = w.copy()
            w /= w.sum(axis=1, keepdims=True)
            absv = np.abs(vv[b, h])
            f = (1 + 2.0 ** -4) * np.exp(2 * eps) * (1 + 2.0 ** -20) - 1
            t1 = f[:, None] * (w @ absv) + 2.0 ** -13 * ((r < 2.0 ** -8) @ absv)
            bound[b, h] = t1 + 2.0 ** -8 * (np.abs(o_ref[b, h]) + t1) + 1e-30
            eps_all[b, h] = eps
    return bound, eps_all


def check_backward(B, H, N, d, dtype, seed, dev, dist="normal", label=""):
    """Run the fused forward and fa_bwd on seeded inputs and hold dQ, dK, dV
    to the bars of tests/test_gpu_backward.py's docstring against the fp64
    gradient oracle.  Returns {name: (rel_f, max_abs / max|ref|)}."""
    q, k, v = make_qkv(B, H, N, d, dtype, seed_base=seed, dist=dist)
    g = torch.Generator().manual_seed(seed + 7)
    do = torch.randn((B, H, N, d), generator=g).to(q.dtype)
    scale = default_scale(d)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = iofa.forward(qd, kd, vd, scale)
    dq, dk, dv = iofa.backward(qd, kd, vd, o, lse, dod, scale)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(widen(q), widen(k), widen(v), widen(do),
                                    float(np.float32(scale)))
    u = UNIT_ROUNDOFF[q.dtype]
    out = {}
    qw, kw, vw, dw = widen(q), widen(k), widen(v), widen(do)
    sum_err = 4 * d * 2.0 ** -24 * np.abs(dw).max() * np.abs(vw).max()
    zero_bound = {"dq": sum_err * scale * np.abs(kw).max(),
                  "dk": sum_err * scale * np.abs(qw).max(), "dv": 0.0}
    for name, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        gw = widen(got.cpu())
        assert np.isfinite(gw).all(), name
        if np.abs(r).max() == 0:
            print(f"{label} {name}: exact zero, max|got|={np.abs(gw).max():.3e} "
                  f"(<= {zero_bound[name]:.2e})", flush=True)
            assert np.abs(gw).max() <= zero_bound[name], (label, name)
            continue
        relf = np.linalg.norm(gw - r) / np.linalg.norm(r)
        rmax = np.abs(gw - r).max() / np.abs(r).max()
        out[name] = (relf, rmax)
        print(f"{label} {name}: rel_f={relf:.3e} (<= {3 * u:.2e}) "
              f"max_abs/max|ref|={rmax:.3e} (<= {12 * u:.2e})", flush=True)
        assert relf <= 3 * u, (label, name, relf)
        assert rmax <= 12 * u, (label, name, rmax)
    return out
