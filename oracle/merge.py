"""Attention over a subset of keys and the merge of such partial results,
fp64 -- TEST INFRASTRUCTURE ONLY (see the package docstring for who may
import it).

[jiahao] "增量求解 softmax" shows that the softmax of a vector split into
blocks p1, p2 follows from each block's local quantities: the global maximum
m(x) = max(m(p1), m(p2)); each block's f and l rescaled by e^{m(pk) - m(x)};
l(x) the sum of the rescaled l's; each block's local softmax weighted by
l(pk)^global / l(x).  Applied to attention with the keys split into G
blocks, every block g yields a partial output O_g (the block's own softmax
over its keys applied to its values) and its log-sum-exp
LSE_g = m_g + ln l_g; then, for every query row,

    LSE = ln sum_g e^{LSE_g}
    O   = sum_g e^{LSE_g - LSE} O_g

because e^{LSE_g - LSE} = e^{m_g - m} l_g / l = l(p_g)^global / l(x).  A block
with no keys has LSE_g = -inf and O_g = 0, and contributes nothing; a row all
of whose blocks are empty therefore sums no terms: LSE = ln 0 = -inf and
O = 0.

``partial_attention`` is the plain definition restricted to a key range; it
uses the same per-head steps as ``standard_attention``.  ``merge_partials`` is the
merge above, written with the largest LSE_g as the reference so that no
exponential overflows.
"""

import numpy as np

from .attention import _rows_of_head


def partial_attention(q, k, v, scale, kv_begin, kv_end):
    """Attention of every query row over keys kv_begin .. kv_end-1 only.

    q: (B, H, Nq, d); k, v: (B, H, Nk, d) / (B, H, Nk, dv).  Returns (O_g,
    LSE_g) of shapes (B, H, Nq, dv) and (B, H, Nq); an empty key range gives
    O_g = 0 and LSE_g = -inf.  The arithmetic is the six steps of
    ``standard_attention`` applied to the key subset.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, _ = q.shape
    o = np.zeros((B, H, Nq, v.shape[3]))
    lse = np.full((B, H, Nq), -np.inf)
    if kv_end <= kv_begin:
        return o, lse
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = _rows_of_head(q[b, h], k[b, h, kv_begin:kv_end],
                                               v[b, h, kv_begin:kv_end], float(scale))
    return o, lse


def merge_partials(o_parts, lse_parts):
    """Merge G partial results: o_parts (G, ..., dv), lse_parts (G, ...).

    Returns (O, LSE) with LSE = ln sum_g e^{LSE_g}, O = sum_g e^{LSE_g - LSE} O_g.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    ref = lse_parts.max(axis=0)                          # largest block LSE
    safe = np.where(np.isfinite(ref), ref, 0.0)
    w = np.exp(lse_parts - safe)                         # e^{LSE_g - ref}, 0 for -inf
    total = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = safe + np.log(total)                       # -inf where every block is empty
    weights = np.divide(w, total, out=np.zeros_like(w), where=total > 0)
    o = (weights[..., None] * o_parts).sum(axis=0)
    return o, lse
