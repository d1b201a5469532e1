"""Tiled attention with the online-softmax recurrence, fp64, with an HBM
element-traffic count -- TEST INFRASTRUCTURE ONLY.

The algorithm of [ctyun] "核心思想" (split the matrices into blocks that fit
on chip) combined with the block form of [xinc] "7. Online Softmax" (keep the
running maximum m, denominator l and un-normalised output z per query row;
one block of scores at a time rescales the old l and z by e^{m_old - m_new}
and adds the new terms; finally o = z / l).  [xinc] "6. 标准注意力为什么慢"
states the result is still exact attention; tests check that against
``standard_attention`` for many block shapes.

Two loop orders are offered:

* ``order="q_outer"``: a Q block stays on chip while every K/V block streams
  past it; m, l, z never leave the chip.  Traffic (elements):
  Q: N*d, K and V: 2*N*d*ceil(N/Br), O: N*dv written, LSE: N written.
* ``order="kv_outer"``: the order [ctyun] "FA MAC分析" analyses -- K/V
  blocks in the outer loop, Q blocks in the inner loop, so Q is re-read once
  per outer step (T_c = ceil(N/Bc) times) and the per-row state z, m, l is
  read and written back each outer step; a last pass forms O = z / l.
  [ctyun] counts only the dominant Q term (N*d*T_c) and drops constants.

The count is in elements ("per float" in [ctyun] "MAC分析"); one LSE value
counts as one element.  Operates on a single head; ``tiled_online_attention``
loops over (B, H).
"""

import math

import numpy as np


def _block_update(state, s_blk, v_blk):
    """One block step of the online recurrence for a slab of rows.

    state = (m, l, z) with shapes (r,), (r,), (r, dv).  s_blk: (r, c) scores,
    v_blk: (c, dv).  Returns the new state.
    """
    m, l, z = state
    m_new = np.maximum(m, s_blk.max(axis=1))
    sub = np.where(m_new == -np.inf, 0.0, m_new)        # -inf guard
    alpha = np.where(m == -np.inf, 0.0, np.exp(m - sub))
    e = np.exp(s_blk - sub[:, None])
    l_new = alpha * l + e.sum(axis=1)
    z_new = alpha[:, None] * z + e @ v_blk
    return m_new, l_new, z_new


def _head_q_outer(q, k, v, scale, br, bc, count):
    n, dv = q.shape[0], v.shape[1]
    o = np.empty((n, dv))
    lse = np.empty(n)
    for i0 in range(0, n, br):
        i1 = min(n, i0 + br)
        qi = q[i0:i1]
        count["Q"] += qi.size
        state = (np.full(i1 - i0, -np.inf), np.zeros(i1 - i0),
                 np.zeros((i1 - i0, dv)))
        for j0 in range(0, n, bc):
            j1 = min(n, j0 + bc)
            kj, vj = k[j0:j1], v[j0:j1]
            count["K"] += kj.size
            count["V"] += vj.size
            state = _block_update(state, scale * (qi @ kj.T), vj)
        m, l, z = state
        o[i0:i1] = z / l[:, None]
        lse[i0:i1] = m + np.log(l)
        count["O"] += (i1 - i0) * dv
        count["LSE"] += i1 - i0
    return o, lse


def _head_kv_outer(q, k, v, scale, br, bc, count):
    n, dv = q.shape[0], v.shape[1]
    # per-row state living in "HBM" between outer steps
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    z = np.zeros((n, dv))
    for j0 in range(0, n, bc):
        j1 = min(n, j0 + bc)
        kj, vj = k[j0:j1], v[j0:j1]
        count["K"] += kj.size
        count["V"] += vj.size
        for i0 in range(0, n, br):
            i1 = min(n, i0 + br)
            qi = q[i0:i1]
            count["Q"] += qi.size
            count["state_read"] += (i1 - i0) * (dv + 2)
            m[i0:i1], l[i0:i1], z[i0:i1] = _block_update(
                (m[i0:i1], l[i0:i1], z[i0:i1]), scale * (qi @ kj.T), vj)
            count["state_write"] += (i1 - i0) * (dv + 2)
    count["state_read"] += n * (dv + 2)        # final pass reads z, m, l
    count["O"] += n * dv
    count["LSE"] += n
    return z / l[:, None], m + np.log(l)


def tiled_online_attention(q, k, v, scale, br, bc, order="q_outer"):
    """Blockwise exact attention over (B, H, N, d) arrays.

    Returns (O, LSE, count) where count maps "Q", "K", "V", "O", "LSE",
    "state_read", "state_write" to element totals over all heads.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if br < 1 or bc < 1:
        raise ValueError("block sizes must be >= 1")
    head = {"q_outer": _head_q_outer, "kv_outer": _head_kv_outer}[order]
    B, H, N, _ = q.shape
    o = np.empty((B, H, N, v.shape[3]))
    lse = np.empty((B, H, N))
    count = dict.fromkeys(["Q", "K", "V", "O", "LSE", "state_read",
                           "state_write"], 0)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = head(q[b, h], k[b, h], v[b, h], float(scale),
                                      br, bc, count)
    return o, lse, count


def q_outer_traffic_elements(n, d, dv, br):
    """Closed form of the q_outer count for one head (elements)."""
    return n * d + 2 * n * d * math.ceil(n / br) + n * dv + n
