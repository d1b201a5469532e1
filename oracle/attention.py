"""Standard (exact) attention in fp64 -- the definition the fused path must reach.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

What is computed, per batch b and head h, for query row i (the three-step
definition of [xinc] "6. 标准注意力为什么慢": S = QK^T/sqrt(d), P = Softmax(S),
O = PV; the same three steps are listed in [jiahao] "Standard Attention" and
[ctyun] "MAC分析 / 标准Transformer MAC分析"):

  1. s_ij = scale * sum_c q_ic k_jc        (the full score row is materialised)
  2. m_i  = max_j s_ij                     ([jiahao] "增量求解 softmax": m)
  3. f_ij = exp(s_ij - m_i), l_i = sum_j f_ij         (f and l)
  4. p_ij = f_ij / l_i                     (s = softmax; the full P row exists)
  5. o_ic = sum_j p_ij v_jc
  6. lse_i = m_i + ln l_i

``scale`` is a caller argument: the pages fix it to 1/sqrt(d); callers pass
the exact fp32 value the GPU receives, widened to fp64.  The log-sum-exp in
step 6 is the "few statistics" that [xinc] "7. Online Softmax" says a backward
pass keeps; it is reported in natural-log units of the scaled scores.

Inputs are widened to fp64 exactly.  16-bit and 32-bit inputs arrive as raw
bit patterns and are decoded here from the IEEE-754 field definitions, so the
oracle relies on no dtype conversion of the GPU side's toolchain.

Row chunking below only bounds memory (a (chunk x N) slab of S and P per
step); every row is computed by the same six steps, independently of the
others.
"""

import numpy as np


def _decode_fields(bits, exp_bits, man_bits):
    """Decode IEEE-754 binary interchange values from their bit fields.

    value = (-1)^s * 2^(e - bias) * (1 + f / 2^man_bits)   for 0 < e < emax
          = (-1)^s * 2^(1 - bias) * (f / 2^man_bits)       for e == 0
          = +-inf (f == 0) or NaN (f != 0)                 for e == emax
    """
    b = np.asarray(bits).astype(np.uint64)
    bias = (1 << (exp_bits - 1)) - 1
    emax = (1 << exp_bits) - 1
    sign = (b >> np.uint64(exp_bits + man_bits)) & np.uint64(1)
    e = ((b >> np.uint64(man_bits)) & np.uint64(emax)).astype(np.int64)
    f = (b & np.uint64((1 << man_bits) - 1)).astype(np.float64)
    frac = f / float(1 << man_bits)
    normal = np.ldexp(1.0 + frac, (e - bias).astype(np.int32))
    subnormal = np.ldexp(frac, 1 - bias)
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where(e == emax, np.where(f == 0, np.inf, np.nan), mag)
    return np.where(sign == 1, -mag, mag)


def decode_bf16(bits):
    """bfloat16 bit patterns (uint16) -> fp64.  Fields: 1 sign, 8 exponent
    (bias 127), 7 mantissa -- the upper half of an IEEE binary32."""
    return _decode_fields(np.asarray(bits, dtype=np.uint16), 8, 7)


def decode_f16(bits):
    """IEEE binary16 bit patterns (uint16) -> fp64.  Fields: 1 sign,
    5 exponent (bias 15), 10 mantissa."""
    return _decode_fields(np.asarray(bits, dtype=np.uint16), 5, 10)


def decode_f32(bits):
    """IEEE binary32 bit patterns (uint32) -> fp64.  Fields: 1 sign,
    8 exponent (bias 127), 23 mantissa."""
    return _decode_fields(np.asarray(bits, dtype=np.uint32), 8, 23)


def _rows_of_head(qh, kh, vh, scale):
    """Steps 1-6 for a slab of query rows ``qh`` against one head's K, V."""
    s = scale * (qh @ kh.T)                    # step 1: S rows, materialised
    m = s.max(axis=1, keepdims=True)           # step 2
    f = np.exp(s - m)                          # step 3
    l = f.sum(axis=1, keepdims=True)
    p = f / l                                  # step 4: P rows, materialised
    o = p @ vh                                 # step 5
    lse = (m + np.log(l))[:, 0]                # step 6
    return o, lse


def _check(q, k, v):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or k.shape[:3] != q.shape[:3] or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k, v must be (B, H, N, d) with matching B, H, N")
    if k.shape[3] != q.shape[3]:
        raise ValueError("q and k must share the head dimension")
    return q, k, v


def standard_attention(q, k, v, scale, row_chunk=1024):
    """Exact attention over (B, H, N, d) fp64 arrays.

    Returns (O, LSE): O is (B, H, N, dv) fp64, LSE is (B, H, N) fp64.
    """
    q, k, v = _check(q, k, v)
    B, H, N, _ = q.shape
    o = np.empty((B, H, N, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    scale = float(scale)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, row_chunk):
                r1 = min(N, r0 + row_chunk)
                o[b, h, r0:r1], lse[b, h, r0:r1] = _rows_of_head(
                    q[b, h, r0:r1], k[b, h], v[b, h], scale)
    return o, lse


def standard_attention_rows(q, k, v, scale, rows):
    """The same definition evaluated only for the query indices ``rows`` of
    every (b, h) -- used to check full-size outputs on a sample of rows.

    Returns (O_rows, LSE_rows) of shapes (B, H, len(rows), dv), (B, H, len(rows)).
    """
    q, k, v = _check(q, k, v)
    rows = np.asarray(rows, dtype=np.int64)
    B, H = q.shape[:2]
    o = np.empty((B, H, rows.size, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, rows.size), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = _rows_of_head(q[b, h, rows], k[b, h], v[b, h],
                                               float(scale))
    return o, lse
