"""Gradients of exact attention, fp64 -- TEST INFRASTRUCTURE ONLY (see the
package docstring for who may import it).

[xinc] "7. Online Softmax" closes by noting that the backward pass reuses the
saved inputs and a few statistics (here the log-sum-exp) to recompute local
scores instead of reading a stored attention matrix.  The quantity it
computes is the plain derivative of standard attention O = P V with
P = Softmax(S), S = scale * Q K^T ([xinc] "6. 标准注意力为什么慢"); for an
upstream gradient dO:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_c dO_ic O_ic            (= sum_j P_ij dP_ij)
    dS = P * (dP - D)                 (softmax Jacobian, row by row)
    dQ = scale * dS K
    dK = scale * dS^T Q

The oracle materialises S, P, dP and dS per head (the plain definition; the
GPU side recomputes them tile by tile from Q, K and the saved LSE).
"""

import numpy as np


def attention_backward(q, k, v, do, scale):
    """(B, H, N, d) fp64 arrays q, k, v, do.  Returns (dq, dk, dv, D) with D
    of shape (B, H, N)."""
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    B, H, N, _ = q.shape
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    Dall = np.empty((B, H, N))
    scale = float(scale)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)          # S
            m = s.max(axis=1, keepdims=True)
            f = np.exp(s - m)
            p = f / f.sum(axis=1, keepdims=True)       # P
            o = p @ v[b, h]                            # O
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T                  # dP
            D = (do[b, h] * o).sum(axis=1)
            ds = p * (dp - D[:, None])                 # dS
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
            Dall[b, h] = D
    return dq, dk, dv, Dall
