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


_WORKLOAD_ORACLE = {}


def workload_oracle(index):
    """The oracle's (O, LSE) over every element of named workload ``index``,
    computed once per process (the fused and the naive tests share it)."""
    if index not in _WORKLOAD_ORACLE:
        from workloads import workload_qkv
        q, k, v, scale, _ = workload_qkv(index)
        _WORKLOAD_ORACLE[index] = oracle_full(q, k, v, scale)
    return _WORKLOAD_ORACLE[index]


def nan_outputs(q, dev):
    """O (q's shape and dtype) and LSE ((B, H, N) fp32) on the device, filled
    with NaN, so any element a kernel fails to write fails the comparison."""
    B, H, N, _ = q.shape
    o = torch.full(q.shape, float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    return o, lse


def sample_rows(N, seed=0, edge=64, middle=64):
    """Query rows checked at full size: the first and last ``edge`` rows (the
    first and the ragged last tiles) plus ``middle`` seeded random rows."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(edge, N))) | set(range(max(0, N - edge), N))
    rows |= set(rng.integers(0, N, size=middle).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def fp8_output_bound(q8, k8, v8, scale, sq, sk, sv, o_ref, rows=None, chunk=1024):
    """Per-element bar on O and per-row score-error bound eps of the FP8
    forward (derivation in tests/test_gpu_fp8.py's docstring), for the rows
    ``rows`` of every head, or all rows.  q8, k8, v8: CPU uint8 code
    tensors; o_ref: the oracle's output for those rows.  Rows are taken in
    chunks of ``chunk`` so a full-size head needs only a (chunk x N) slab."""
    qd, kd, vd = (oracle.decode_e4m3(t.numpy()) for t in (q8, k8, v8))
    qv, kv, vv = oracle.fp8_values(q8.numpy(), k8.numpy(), v8.numpy(), sq, sk, sv)
    if rows is not None:
        qd, qv = qd[:, :, rows], qv[:, :, rows]
    c = abs(float(np.float32(scale))) * float(np.float32(sq)) * float(np.float32(sk))
    B, H, R = qd.shape[:3]
    bound = np.empty_like(o_ref)
    eps_all = np.empty(o_ref.shape[:3])
    for b in range(B):
        for h in range(H):
            absk = np.abs(kd[b, h]).T
            absv = np.abs(vv[b, h])
            for r0 in range(0, R, chunk):
                r1 = min(R, r0 + chunk)
                mag = np.abs(qd[b, h, r0:r1]) @ absk                # sum_c |q8 k8|
                s = float(np.float32(scale)) * (qv[b, h, r0:r1] @ kv[b, h].T)
                eps = 2.0 ** -10 * c * mag.max(axis=1) + 2.0 ** -20 * (1 + np.abs(s).max(axis=1))
                del mag
                w = np.exp(s - s.max(axis=1, keepdims=True))
                small = (w < 2.0 ** -8) @ absv
                w /= w.sum(axis=1, keepdims=True)
                f = (1 + 2.0 ** -4) * np.exp(2 * eps) * (1 + 2.0 ** -20) - 1
                t1 = f[:, None] * (w @ absv) + 2.0 ** -13 * small
                bound[b, h, r0:r1] = t1 + 2.0 ** -8 * (np.abs(o_ref[b, h, r0:r1]) + t1) + 1e-30
                eps_all[b, h, r0:r1] = eps
    return bound, eps_all


def naive_output_bound(q, k, v, scale, o_ref, lse_ref, rows=None, chunk=512):
    """Per-element bar on O and per-row bar on LSE of the naive three-kernel
    path for 16-bit inputs, which stores S and P in the input type
    (u = 2^-8 for bf16, 2^-11 for fp16).  Derived from its arithmetic:

    * K1 forms s_j = scale * q.k_j with fp32 accumulation (error at most
      (d + 2) 2^-24 |scale| sum_c |q_c k_jc|) and rounds it to the input type
      (u |s_j|); the fp32 exponent arithmetic of K2 adds at most
      2^-20 (2 + |s_j| + max_k |s_k|).  Call the sum delta_j: the stored score
      is s_j + Delta_j with |Delta_j| <= delta_j.
    * The stored weights are then proportional to w_j e^{Delta_j} (w the
      exact softmax), so after normalisation each changes by a factor within
      e^{+-(delta_j + D)}, where D = ln sum_j w_j e^{delta_j} bounds the shift
      of the log-sum-exp (Jensen, both directions).
    * K2's fp32 row sum (N 2^-24 relative), division and the rounding of P to
      the input type (u) scale each weight by at most 1 + eps_p more,
      eps_p = u + (N + 4) 2^-24.
    * K3 accumulates sum_j p_j v_jc in fp32 (N 2^-24 of sum_j p_j |v_jc|) and
      rounds O to the input type (u |O|).

    So |O_c - O_ref_c| <= A_c + u (|O_ref_c| + A_c) with
    A_c = sum_j w_j |v_jc| ((1 + eps_p)(1 + N 2^-24) e^{delta_j + D} - 1), and
    |LSE - LSE_ref| <= D + (N + 8) 2^-24 + 2^-20 (1 + |LSE_ref|).
    Returns (bound on O, bound on LSE) for the rows ``rows`` of every head
    (or all rows); o_ref, lse_ref are the oracle's values for those rows."""
    u = UNIT_ROUNDOFF[q.dtype]
    qw, kw, vw = widen(q), widen(k), widen(v)
    if rows is not None:
        qw = qw[:, :, rows]
    B, H, R, d = qw.shape
    N = kw.shape[2]
    sc = abs(float(np.float32(scale)))
    eps_p = u + (N + 4) * 2.0 ** -24
    grow = (1 + eps_p) * (1 + N * 2.0 ** -24)
    bound = np.empty_like(o_ref)
    lbound = np.empty(o_ref.shape[:3])
    for b in range(B):
        for h in range(H):
            kt, absk = kw[b, h].T, np.abs(kw[b, h]).T
            absv = np.abs(vw[b, h])
            for r0 in range(0, R, chunk):
                r1 = min(R, r0 + chunk)
                s = float(np.float32(scale)) * (qw[b, h, r0:r1] @ kt)
                acc = (d + 2) * 2.0 ** -24 * sc * (np.abs(qw[b, h, r0:r1]) @ absk)
                smax = np.abs(s).max(axis=1, keepdims=True)
                delta = u * np.abs(s) + acc + 2.0 ** -20 * (2 + np.abs(s) + smax)
                del acc
                w = np.exp(s - lse_ref[b, h, r0:r1, None])      # exact softmax weights
                del s
                dsh = np.log((w * np.exp(delta)).sum(axis=1))   # D per row
                wf = w * (grow * np.exp(delta + dsh[:, None]) - 1)
                a = wf @ absv
                bound[b, h, r0:r1] = a + u * (np.abs(o_ref[b, h, r0:r1]) + a) + 1e-30
                lbound[b, h, r0:r1] = (dsh + (N + 8) * 2.0 ** -24
                                       + 2.0 ** -20 * (1 + np.abs(lse_ref[b, h, r0:r1])))
    return bound, lbound


def tile_rows(N, H, seed, per_tile=2, tile=128):
    """Query rows to check at full size, a different set for each of the H
    heads: ``per_tile`` distinct seeded random rows inside every ``tile``-row
    query tile, always including the sequence's first and last rows.
    Returns an (H, R) array of sorted rows."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(H):
        rows = []
        for t0 in range(0, N, tile):
            t1 = min(N, t0 + tile)
            forced = [r for r in (0, N - 1) if t0 <= r < t1]
            pool = np.setdiff1d(np.arange(t0, t1), forced)
            k = min(per_tile, t1 - t0) - len(forced)
            rows += forced + rng.choice(pool, size=max(k, 0), replace=False).tolist()
        out.append(sorted(rows))
    return np.array(out, dtype=np.int64)


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
