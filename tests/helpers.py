"""Shared test helpers: running the oracle on the exact inputs the GPU sees,
tolerances, and comparisons."""

import numpy as np
import torch

import oracle
from workloads import raw_bits

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
