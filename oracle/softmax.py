"""Softmax in the pages' incremental forms, fp64 -- TEST INFRASTRUCTURE ONLY.

Three forms of one result:

* ``local_softmax`` -- the per-block quantities m, f, l, s of [jiahao]
  "增量求解 softmax" (the safe two-pass softmax of one block).
* ``two_block_softmax`` -- the same section's merge of two blocks p1, p2 into
  the global softmax: m(x) = max(m(p1), m(p2)); each block's f and l are
  rescaled by e^{m(pk) - m(x)}; l(x) is the sum of the rescaled l's; each
  block's local softmax is scaled by l(pk)^global / l(x).
* ``online_softmax_output`` -- [xinc] "7. Online Softmax": running maximum
  m_t, denominator l_t and un-normalised weighted sum z_t of value rows; a
  new score (or, as that section allows, a block of scores) rescales the old
  l and z by e^{m_t - m_{t+1}} and adds the new terms; o = z_N / l_N.

Readings of garbled formulas on [jiahao] "增量求解 softmax":
  * f(p2) and l(p2) are printed with m(p1) in the exponent and the l(p2)
    update sums i = k+1 .. k; the right-hand sides of those same lines
    (l(p2) * e^{m(p2) - m(x)}) fix the intended m(p2) and upper limit n.
  * s(pk)^global is printed as l(pk)^global / l(x) with a note that it is
    broadcast; read as s(pk) * l(pk)^global / l(x), which equals
    e^{x_i - m(x)} / l(x) for every element of block k.

Empty or fully masked blocks (and the initial state of the online form) use
m = -inf, l = 0, z = 0, and a local softmax of zeros.  Where the new running maximum is still -inf (only -inf scores seen so
far) the subtrahend is taken as 0 so that no NaN appears.
"""

import numpy as np


def local_softmax(x):
    """Block statistics of [jiahao] "增量求解 softmax": returns (m, f, l, s)."""
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0 or x.max() == -np.inf:
        # empty or fully masked block: it contributes nothing (m = -inf, l = 0,
        # and its local softmax is taken as all zeros instead of 0/0)
        return -np.inf, np.zeros_like(x), 0.0, np.zeros_like(x)
    m = x.max()
    f = np.exp(x - m)
    l = f.sum()
    return m, f, l, f / l


def _rescale(m_old, m_new):
    """e^{m_old - m_new}, with the -inf guard described in the module doc."""
    if m_old == -np.inf:
        return 0.0
    return np.exp(m_old - m_new)


def two_block_softmax(x, k):
    """Global softmax of x from the local softmaxes of p1 = x[:k], p2 = x[k:].

    Returns (softmax(x), m(x), l(x), f_global) where f_global is the
    concatenation of f(p1)^global and f(p2)^global (= e^{x - m(x)}).
    """
    x = np.asarray(x, dtype=np.float64)
    m1, f1, l1, s1 = local_softmax(x[:k])
    m2, f2, l2, s2 = local_softmax(x[k:])
    m = max(m1, m2)                              # m(x)
    a1 = _rescale(m1, m)                         # e^{m(p1) - m(x)}
    a2 = _rescale(m2, m)                         # e^{m(p2) - m(x)}
    f1g, f2g = f1 * a1, f2 * a2                  # f(pk)^global
    l1g, l2g = l1 * a1, l2 * a2                  # l(pk)^global
    l = l1g + l2g                                # l(x)
    s1g = s1 * (l1g / l)                         # s(pk)^global (broadcast)
    s2g = s2 * (l2g / l)
    return np.concatenate([s1g, s2g]), m, l, np.concatenate([f1g, f2g])


def online_softmax_output(s, v, block=1):
    """Online softmax-weighted average of value rows.

    s: (n,) scores; v: (n, dv) value rows; scores are added ``block`` at a
    time.  Returns (o, m_N, l_N) with o = z_N / l_N.
    """
    s = np.asarray(s, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = s.shape[0]
    m = -np.inf
    l = 0.0
    z = np.zeros(v.shape[1:], dtype=np.float64)
    for t0 in range(0, n, block):
        sb = s[t0:t0 + block]
        vb = v[t0:t0 + block]
        m_new = max(m, sb.max())                 # m_{t+1} = max(m_t, s_{t+1})
        sub = 0.0 if m_new == -np.inf else m_new
        alpha = _rescale(m, m_new)               # e^{m_t - m_{t+1}}
        e = np.exp(sb - sub)                     # e^{s_{t+1} - m_{t+1}}
        l = alpha * l + e.sum()                  # l_{t+1}
        z = alpha * z + e @ vb                   # z_{t+1}
        m = m_new
    return z / l, m, l


def softmax_rows(x):
    """Row-wise softmax of a 2-D array by the per-block quantities of
    [jiahao] "增量求解 softmax" taken over the whole row (one block):
    returns (y, lse) with y[r] = s(row r) and lse[r] = m + ln l."""
    x = np.asarray(x, dtype=np.float64)
    y = np.empty_like(x)
    lse = np.empty(x.shape[0])
    for r in range(x.shape[0]):
        m, _, l, s = local_softmax(x[r])
        y[r] = s
        lse[r] = m + np.log(l) if l > 0 else -np.inf
    return y, lse


def online_row_stats(x, block):
    """Running maximum and denominator of one row, adding ``block`` scores at
    a time ([xinc] "7. Online Softmax": a new block rescales the old l by
    e^{m_old - m_new} and adds its own terms).  Returns (m, l)."""
    x = np.asarray(x, dtype=np.float64)
    m, l = -np.inf, 0.0
    for t0 in range(0, x.shape[0], block):
        xb = x[t0:t0 + block]
        m_new = max(m, xb.max())
        if m_new == -np.inf:
            continue
        l = _rescale(m, m_new) * l + np.exp(xb - m_new).sum()
        m = m_new
    return m, l
