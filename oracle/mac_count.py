"""Element-access count of standard three-step attention -- TEST INFRASTRUCTURE.

A CPU mirror of the three steps of standard attention that [ctyun]
"MAC分析 / 标准Transformer MAC分析" analyses, run against a counting stand-in
for HBM.  Each step loads its input matrices from the stand-in once and stores
its output once, exactly as that section assumes ("per float" accessed):

  first step:  read Q, K; S = scale * Q K^T; write S
  second step: read S; P = softmax(S) (row-wise, safe form); write P
  third step:  read P, V; O = P V; write O

The page's per-step totals (2Nd + N^2, 2N^2, N^2 + 2Nd; sum 4Nd + 4N^2) are
pinned by a test against these counts; the arithmetic is the same definition
as ``standard_attention`` and is checked against it.  The initial placement
of Q, K, V in the stand-in is not counted (the inputs are already resident).
"""

import numpy as np


class CountingHBM:
    """Dictionary of named matrices that counts elements read and written."""

    def __init__(self):
        self._mem = {}
        self.reads = 0
        self.writes = 0

    def place(self, name, arr):
        """Make an input resident without counting it."""
        self._mem[name] = np.array(arr, dtype=np.float64)

    def read(self, name):
        arr = self._mem[name]
        self.reads += arr.size
        return arr.copy()

    def write(self, name, arr):
        arr = np.array(arr, dtype=np.float64)
        self.writes += arr.size
        self._mem[name] = arr


def standard_attention_mac(q, k, v, scale):
    """One head: q, k (N, d), v (N, dv).  Returns (O, per_step) where
    per_step is a list of three (reads, writes) element counts."""
    hbm = CountingHBM()
    hbm.place("Q", q)
    hbm.place("K", k)
    hbm.place("V", v)
    per_step = []

    r0, w0 = hbm.reads, hbm.writes
    qm, km = hbm.read("Q"), hbm.read("K")
    hbm.write("S", scale * (qm @ km.T))
    per_step.append((hbm.reads - r0, hbm.writes - w0))

    r0, w0 = hbm.reads, hbm.writes
    s = hbm.read("S")
    f = np.exp(s - s.max(axis=1, keepdims=True))
    hbm.write("P", f / f.sum(axis=1, keepdims=True))
    per_step.append((hbm.reads - r0, hbm.writes - w0))

    r0, w0 = hbm.reads, hbm.writes
    p, vm = hbm.read("P"), hbm.read("V")
    hbm.write("O", p @ vm)
    per_step.append((hbm.reads - r0, hbm.writes - w0))

    return hbm.read("O"), per_step
