"""Pins of the fp64 oracle against things other than itself.

Each check compares the oracle with an independent source of truth: 40-digit
decimal brute force on tiny inputs, closed forms, invariants of the
definition, library dtype conversions, and the element counts printed on the
ctyun.cn FlashAttention article (section "MAC分析").  ``test_planted_mistakes``
plants plausible mistakes into a copy of the oracle's row computation and
shows that at least one pin fails for each.
"""

import decimal
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oatt
from oracle.tiled import q_outer_traffic_elements

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = decimal.Decimal


# ----------------------------------------------------------------- decoders

def test_decode_bf16_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle.decode_bf16(bits)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()


def test_decode_f16_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.decode_f16(bits)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()


def test_decode_f32_sampled_patterns():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    specials = np.array([0, 0x80000000, 1, 0x807FFFFF, 0x00800000, 0x7F7FFFFF,
                         0x7F800000, 0xFF800000, 0x7FC00000, 0x3F800000],
                        dtype=np.uint32)
    bits = np.concatenate([bits, specials])
    with np.errstate(invalid="ignore"):
        ref = bits.view(np.float32).astype(np.float64)
    got = oracle.decode_f32(bits)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()


# ------------------------------------------------------- decimal brute force

def brute_attention(q, k, v, scale, prec=40):
    """Attention by its definition in 40-digit decimal arithmetic, with no max
    subtraction and plain left-to-right sums.  q, k: (N, d); v: (N, dv)."""
    ctx = decimal.Context(prec=prec)
    n, d = q.shape
    dv = v.shape[1]
    sc = D(float(scale))
    o = np.empty((n, dv))
    lse = np.empty(n)
    for i in range(n):
        e = []
        for j in range(n):
            acc = D(0)
            for c in range(d):
                acc = ctx.add(acc, ctx.multiply(D(float(q[i, c])), D(float(k[j, c]))))
            e.append(ctx.exp(ctx.multiply(sc, acc)))
        l = D(0)
        for x in e:
            l = ctx.add(l, x)
        for c in range(dv):
            acc = D(0)
            for j in range(n):
                acc = ctx.add(acc, ctx.multiply(ctx.divide(e[j], l), D(float(v[j, c]))))
            o[i, c] = float(acc)
        lse[i] = float(ctx.ln(l))
    return o, lse


def brute_softmax(x, prec=40):
    ctx = decimal.Context(prec=prec)
    e = [D(0) if xi == -np.inf else ctx.exp(D(float(xi))) for xi in x]
    l = D(0)
    for t in e:
        l = ctx.add(l, t)
    return np.array([float(ctx.divide(t, l)) for t in e]), l


def _tiny_case(seed, n, d, dv=None, spread=1.0):
    rng = np.random.default_rng(seed)
    dv = d if dv is None else dv
    q = rng.normal(size=(n, d)) * spread
    k = rng.normal(size=(n, d)) * spread
    v = rng.normal(size=(n, dv))
    return q, k, v


def _oracle_one_head(q, k, v, scale):
    o, lse = oracle.standard_attention(q[None, None], k[None, None], v[None, None], scale)
    return o[0, 0], lse[0, 0]


def brute_force_pin_holds(attention_fn, cases):
    """True iff ``attention_fn`` agrees with decimal brute force on ``cases``."""
    for seed, n, d, dv, spread, scale in cases:
        q, k, v = _tiny_case(seed, n, d, dv, spread)
        o, lse = attention_fn(q, k, v, scale)
        ob, lb = brute_attention(q, k, v, scale)
        if not (np.allclose(o, ob, rtol=1e-13, atol=1e-13)
                and np.allclose(lse, lb, rtol=1e-13, atol=1e-13)):
            return False
    return True


BRUTE_CASES = [
    (1, 1, 1, 1, 1.0, 1.0),
    (2, 2, 3, 2, 1.0, 0.5),
    (3, 3, 3, 3, 1.5, 0.7),     # N == d == dv: a transposed operand still runs
    (4, 5, 4, 3, 1.0, 0.5),
    (5, 8, 8, 8, 2.0, 1.0 / math.sqrt(8)),
    (6, 16, 8, 4, 1.0, 1.0 / math.sqrt(8)),
    (7, 16, 2, 5, 3.0, 0.9),    # wide score spread: max subtraction matters in fp64
]


def test_brute_force_tiny():
    assert brute_force_pin_holds(_oracle_one_head, BRUTE_CASES)


def test_rows_variant_matches_brute_force():
    q, k, v = _tiny_case(11, 13, 4, 3)
    rows = [0, 5, 12]
    o, lse = oracle.standard_attention_rows(q[None, None], k[None, None], v[None, None], 0.6, rows)
    ob, lb = brute_attention(q, k, v, 0.6)
    np.testing.assert_allclose(o[0, 0], ob[rows], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], lb[rows], rtol=1e-13, atol=1e-13)


# -------------------------------------------------------------- closed forms

def closed_form_pin_holds(attention_fn):
    """Hand-derived cases of the definition."""
    ok = True
    # two keys, one query: scores (0, s); p = (1, e^s) / (1 + e^s)
    for s in (0.0, 1.0, -2.5, 30.0):
        a, b = 0.25, -3.0
        q = np.array([[1.0]])
        k = np.array([[0.0], [1.0]])
        v = np.array([[a], [b]])
        o, lse = attention_fn(q[[0, 0]], k, v, s)
        o_ref = (a + b * math.exp(s)) / (1.0 + math.exp(s))
        lse_ref = math.log1p(math.exp(s)) if s < 20 else s + math.log1p(math.exp(-s))
        ok &= abs(o[0, 0] - o_ref) <= 1e-14 * max(1.0, abs(o_ref))
        ok &= abs(lse[0] - lse_ref) <= 1e-14 * max(1.0, abs(lse_ref))
    # N = 1: O = V exactly, LSE = scale * q.k
    q, k, v = _tiny_case(21, 1, 6, 4)
    o, lse = attention_fn(q, k, v, 0.3)
    ok &= bool(np.array_equal(o, v))
    ok &= abs(lse[0] - 0.3 * float(q[0] @ k[0])) <= 1e-14 * max(1.0, abs(lse[0]))
    # Q = 0: every score is 0, so O_i = mean_j V_j and LSE = ln N
    _, k, v = _tiny_case(22, 9, 4, 3)
    o, lse = attention_fn(np.zeros((9, 4)), k, v, 1.0)
    ok &= bool(np.allclose(o, v.mean(axis=0)[None, :], rtol=0, atol=1e-14))
    ok &= bool(np.allclose(lse, math.log(9), rtol=0, atol=1e-14))
    # asymmetric 2x2 with d=2 and V = I (so O = P): catches a transposed
    # score matrix or a softmax taken down columns
    q = np.array([[2.0, 0.0], [0.0, 3.0]])
    k = np.array([[1.0, 0.0], [0.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    o, lse = attention_fn(q, k, v, 1.0)
    # row 0: scores (2, 0) -> p = (e^2, 1)/(e^2+1); row 1: scores (0, 0) -> p = (1/2, 1/2)
    e2 = math.exp(2.0)
    ok &= bool(np.allclose(o[0], [e2 / (e2 + 1), 1 / (e2 + 1)], rtol=0, atol=1e-14))
    ok &= bool(np.allclose(o[1], [0.5, 0.5], rtol=0, atol=1e-14))
    ok &= abs(lse[0] - math.log(e2 + 1)) <= 1e-14 and abs(lse[1] - math.log(2)) <= 1e-14
    return bool(ok)


def test_closed_forms():
    assert closed_form_pin_holds(_oracle_one_head)


def test_identity_values_give_p_rows_summing_to_one():
    # V = I makes O = P: entries in [0, 1], rows sum to 1; V = ones gives O = 1.
    for seed, n, d in [(31, 7, 3), (32, 40, 16)]:
        q, k, _ = _tiny_case(seed, n, d, spread=2.0)
        p, _ = _oracle_one_head(q, k, np.eye(n), 0.5)
        assert (p >= 0).all() and (p <= 1).all()
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
        ones, _ = _oracle_one_head(q, k, np.ones((n, 5)), 0.5)
        np.testing.assert_allclose(ones, 1.0, rtol=0, atol=1e-13)


def test_shift_invariance():
    # K' = K + 1 u^T shifts row i's scores by scale * q_i . u: O is unchanged
    # and LSE_i moves by exactly that amount.  Values on a 1/8 grid.
    rng = np.random.default_rng(41)
    q = rng.integers(-32, 33, size=(2, 3, 50, 16)) / 8.0
    k = rng.integers(-32, 33, size=(2, 3, 50, 16)) / 8.0
    v = rng.normal(size=(2, 3, 50, 16))
    u = rng.integers(-32, 33, size=16) / 8.0
    scale = 0.25
    o1, l1 = oracle.standard_attention(q, k, v, scale)
    o2, l2 = oracle.standard_attention(q, k + u, v, scale)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, scale * (q @ u), rtol=0, atol=1e-11)


def test_permutation_equivariance():
    rng = np.random.default_rng(42)
    q, k, v = (rng.normal(size=(1, 2, 33, 8)) for _ in range(3))
    o, lse = oracle.standard_attention(q, k, v, 0.4)
    pk = rng.permutation(33)
    o2, lse2 = oracle.standard_attention(q, k[:, :, pk], v[:, :, pk], 0.4)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)
    pq = rng.permutation(33)
    o3, lse3 = oracle.standard_attention(q[:, :, pq], k, v, 0.4)
    np.testing.assert_allclose(o3, o[:, :, pq], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse3, lse[:, :, pq], rtol=0, atol=1e-13)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(43)
    q, k, v = _tiny_case(44, 12, 8)
    j = 7
    k[j] = 60.0 * q[3] / np.linalg.norm(q[3])
    o, _ = _oracle_one_head(q, k, v, 1.0)
    np.testing.assert_allclose(o[3], v[j], rtol=0, atol=1e-12)


def test_batches_and_heads_are_independent():
    rng = np.random.default_rng(45)
    q, k, v = (rng.normal(size=(2, 3, 10, 4)) for _ in range(3))
    o, lse = oracle.standard_attention(q, k, v, 0.5)
    for b in range(2):
        for h in range(3):
            ob, lb = brute_attention(q[b, h], k[b, h], v[b, h], 0.5)
            np.testing.assert_allclose(o[b, h], ob, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(lse[b, h], lb, rtol=1e-13, atol=1e-13)


def test_row_chunking_does_not_change_rows():
    rng = np.random.default_rng(46)
    q, k, v = (rng.normal(size=(1, 1, 37, 4)) for _ in range(3))
    o1, l1 = oracle.standard_attention(q, k, v, 0.5, row_chunk=1024)
    o2, l2 = oracle.standard_attention(q, k, v, 0.5, row_chunk=5)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-15)


# ----------------------------------------- blockwise merge / online recurrence

@pytest.mark.parametrize("n", [1, 2, 3, 7, 16, 32])
def test_two_block_merge_equals_softmax(n):
    rng = np.random.default_rng(100 + n)
    for spread in (1.0, 30.0):
        x = rng.normal(size=n) * spread
        ref, l_ref = brute_softmax(x)
        m_ref = x.max()
        for k in range(0, n + 1):
            s, m, l, f = oracle.two_block_softmax(x, k)
            np.testing.assert_allclose(s, ref, rtol=0, atol=1e-14)
            assert m == m_ref
            # l(x) = sum e^{x - m(x)}; f_global = e^{x - m(x)}
            ctx = decimal.Context(prec=40)
            l_dec = float(ctx.divide(l_ref, ctx.exp(D(float(m_ref)))))
            assert abs(l - l_dec) <= 1e-14 * l_dec
            np.testing.assert_allclose(f / l, ref, rtol=0, atol=1e-14)


def test_two_block_merge_with_masked_block():
    x = np.array([-np.inf, -np.inf, 0.5, 2.0, -1.0])
    for k in range(6):
        s, _, _, _ = oracle.two_block_softmax(x, k)
        ref, _ = brute_softmax(x)
        np.testing.assert_allclose(s, ref, rtol=0, atol=1e-15)
        assert s[0] == 0.0 and s[1] == 0.0


@pytest.mark.parametrize("n", [1, 5, 16, 33])
def test_online_recurrence_equals_weighted_average(n):
    rng = np.random.default_rng(200 + n)
    for spread in (1.0, 25.0):
        s = rng.normal(size=n) * spread
        v = rng.normal(size=(n, 3))
        p, l_ref = brute_softmax(s)
        ctx = decimal.Context(prec=40)
        o_ref = np.array([float(sum((D(float(p[j])) * D(float(v[j, c])) for j in range(n)), D(0)))
                          for c in range(3)])
        for block in sorted({1, 2, 3, n, n + 4}):
            o, m, l = oracle.online_softmax_output(s, v, block=block)
            np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-14)
            assert m == s.max()
            l_dec = float(ctx.divide(l_ref, ctx.exp(D(float(s.max())))))
            assert abs(l - l_dec) <= 1e-13 * l_dec


def test_online_recurrence_masked_prefix():
    # a leading block of -inf scores exercises the -inf guard
    s = np.array([-np.inf, -np.inf, -np.inf, 1.0, 3.0])
    v = np.arange(10, dtype=float).reshape(5, 2)
    for block in (1, 2, 3):
        o, m, l = oracle.online_softmax_output(s, v, block=block)
        w = np.array([math.exp(-2.0), 1.0]) / (1.0 + math.exp(-2.0))
        np.testing.assert_allclose(o, w @ v[3:], rtol=0, atol=1e-14)
        assert m == 3.0 and np.isfinite(l)


# ------------------------------------------------------------ tiled mirror

@pytest.mark.parametrize("order", ["q_outer", "kv_outer"])
@pytest.mark.parametrize("br,bc", [(1, 1), (4, 3), (7, 16), (64, 5), (100, 100)])
def test_tiled_equals_definition(order, br, bc):
    rng = np.random.default_rng(300 + br * 7 + bc)
    q = rng.normal(size=(2, 2, 37, 8)) * 2.0
    k = rng.normal(size=(2, 2, 37, 8)) * 2.0
    v = rng.normal(size=(2, 2, 37, 5))
    o_ref, l_ref = oracle.standard_attention(q, k, v, 0.7)
    o, lse, cnt = oracle.tiled_online_attention(q, k, v, 0.7, br, bc, order=order)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-12)
    n, d, dv, heads = 37, 8, 5, 4
    if order == "q_outer":
        total = cnt["Q"] + cnt["K"] + cnt["V"] + cnt["O"] + cnt["LSE"]
        # K is d wide, V is dv wide
        want = heads * (n * d + n * d * math.ceil(n / br) + n * dv * math.ceil(n / br)
                        + n * dv + n)
        assert total == want
        assert q_outer_traffic_elements(n, d, d, br) == n * d + 2 * n * d * math.ceil(n / br) + n * d + n
    else:
        # the dominant term of the ctyun.cn article's "FA MAC分析": Q read T_c times
        assert cnt["Q"] == heads * n * d * math.ceil(n / bc)
        assert cnt["K"] == heads * n * d and cnt["V"] == heads * n * dv


# -------------------------------------------------------------- MAC count

def _eval(expr, N, d):
    return eval(expr, {"__builtins__": {}}, {"N": N, "d": d})


@pytest.mark.parametrize("N,d", [(1, 1), (5, 3), (16, 8), (33, 4)])
def test_mac_count_matches_printed_formulas(N, d):
    with open(os.path.join(GOLDEN, "mac_standard_attention.json"), encoding="utf-8") as fh:
        g = json.load(fh)
    rng = np.random.default_rng(N * 100 + d)
    q, k, v = (rng.normal(size=(N, d)) for _ in range(3))
    o, per_step = oracle.standard_attention_mac(q, k, v, 0.5)
    for (reads, writes), spec in zip(per_step, g["per_step"]):
        assert reads == sum(_eval(e, N, d) for e in spec["reads"].values())
        assert writes == sum(_eval(e, N, d) for e in spec["writes"].values())
        assert reads + writes == _eval(spec["printed_total"], N, d)
    assert sum(r + w for r, w in per_step) == _eval(g["printed_sum"], N, d)
    transfers = sum(len(s["reads"]) + len(s["writes"]) for s in g["per_step"])
    assert transfers == g["matrix_transfers"]
    o_ref, _ = _oracle_one_head(q, k, v, 0.5)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)


# ------------------------------------------------------- planted mistakes

def _mutant(kind):
    def rows(qh, kh, vh, scale):
        s = scale * (qh @ kh.T)
        if kind == "no_scale":
            s = qh @ kh.T
        if kind == "transposed_scores":
            s = scale * (kh @ qh.T)
        m = s.max(axis=1, keepdims=True)
        f = np.exp(s - m)
        if kind == "sign":
            f = np.exp(m - s)
        l = f.sum(axis=1, keepdims=True)
        if kind == "column_sum":
            l = f.sum(axis=0, keepdims=True)
        p = f / l
        o = p @ vh
        if kind == "transposed_p":
            o = p.T @ vh
        if kind == "dropped_term":
            o = p[:, 1:] @ vh[1:]
        lse = (m + np.log(l))[:, 0] if kind != "lse_no_max" else np.log(l)[:, 0]
        if kind == "column_sum":
            lse = (m + np.log(l[:, :1]))[:, 0]
        return o, lse
    return rows


@pytest.mark.parametrize("kind", ["no_scale", "transposed_scores", "sign", "column_sum",
                                  "transposed_p", "dropped_term", "lse_no_max"])
def test_planted_mistakes_fail_a_pin(kind, monkeypatch):
    monkeypatch.setattr(oatt, "_rows_of_head", _mutant(kind))
    cases = [c for c in BRUTE_CASES if c[1] == c[2] == c[3]] + [BRUTE_CASES[3]]

    def guarded(fn):
        try:
            return fn()
        except (ValueError, IndexError):
            return False     # a shape error is a failed pin too
    held = guarded(lambda: brute_force_pin_holds(_oracle_one_head, cases)) and \
        guarded(lambda: closed_form_pin_holds(_oracle_one_head))
    assert not held, f"mutant {kind!r} passed every pin"


# ------------------------------------------------ partial attention + merge

def _random_head(seed, B=1, H=2, N=37, d=8, dv=5):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d)),
            rng.standard_normal((B, H, N, dv)))


@pytest.mark.parametrize("cuts", [[0, 37], [0, 1, 37], [0, 16, 32, 37], [0, 5, 6, 20, 36, 37],
                                  list(range(0, 38))])
def test_merge_of_key_blocks_equals_definition(cuts):
    # [jiahao] "增量求解 softmax": the blockwise merge reproduces the global
    # softmax; here for attention rows with keys cut at `cuts`
    q, k, v = _random_head(3)
    scale = 0.7
    parts = [oracle.partial_attention(q, k, v, scale, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = oracle.merge_partials(np.stack([p[0] for p in parts]),
                                   np.stack([p[1] for p in parts]))
    o_ref, lse_ref = oracle.standard_attention(q, k, v, scale)
    assert np.abs(o - o_ref).max() <= 1e-13
    assert np.abs(lse - lse_ref).max() <= 1e-13


def test_partial_attention_over_all_keys_is_the_definition():
    q, k, v = _random_head(4)
    o, lse = oracle.partial_attention(q, k, v, 0.3, 0, 37)
    o_ref, lse_ref = oracle.standard_attention(q, k, v, 0.3)
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)


def test_merge_identities():
    q, k, v = _random_head(5)
    a = oracle.partial_attention(q, k, v, 0.5, 0, 20)
    b = oracle.partial_attention(q, k, v, 0.5, 20, 37)
    empty = oracle.partial_attention(q, k, v, 0.5, 7, 7)
    assert np.all(empty[1] == -np.inf) and np.all(empty[0] == 0)
    one = oracle.merge_partials(a[0][None], a[1][None])           # G = 1
    assert np.abs(one[0] - a[0]).max() <= 1e-15 and np.abs(one[1] - a[1]).max() <= 1e-15
    ab = oracle.merge_partials(np.stack([a[0], b[0]]), np.stack([a[1], b[1]]))
    ba = oracle.merge_partials(np.stack([b[0], a[0]]), np.stack([b[1], a[1]]))
    aeb = oracle.merge_partials(np.stack([a[0], empty[0], b[0]]),
                                np.stack([a[1], empty[1], b[1]]))
    for other in (ba, aeb):
        assert np.abs(other[0] - ab[0]).max() <= 1e-14
        assert np.abs(other[1] - ab[1]).max() <= 1e-14


def test_merge_of_rows_without_keys():
    # rows whose blocks are all empty sum no terms (O = 0, LSE = -inf); the
    # other rows are unaffected by an empty block next to them
    q, k, v = _random_head(6)
    a = oracle.partial_attention(q, k, v, 0.5, 0, 37)
    empty = oracle.partial_attention(q, k, v, 0.5, 9, 9)
    o, lse = oracle.merge_partials(np.stack([empty[0], empty[0]]), np.stack([empty[1], empty[1]]))
    assert np.all(o == 0) and np.all(lse == -np.inf)
    o_parts = np.stack([a[0], empty[0]])
    lse_parts = np.stack([a[1], empty[1]])
    lse_parts[0, 0, 0, ::2] = -np.inf               # every other row: both blocks empty
    o_parts[0, 0, 0, ::2] = 0.0
    o, lse = oracle.merge_partials(o_parts, lse_parts)
    assert np.all(o[0, 0, ::2] == 0) and np.all(lse[0, 0, ::2] == -np.inf)
    assert np.abs(o[0, 0, 1::2] - a[0][0, 0, 1::2]).max() <= 1e-15
    assert np.abs(lse[0, 0, 1::2] - a[1][0, 0, 1::2]).max() <= 1e-15


@pytest.mark.parametrize("n", [2, 5, 16])
def test_merge_weights_match_two_block_softmax(n):
    # one query row, V = identity: the output row is the attention weights, so
    # the merge must give the same vector as the two-block formula of
    # [jiahao] "增量求解 softmax" for every split point
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n) * 3
    q = np.ones((1, 1, 1, 1))
    kk = x.reshape(1, 1, n, 1)                 # scores = x with scale 1
    v = np.eye(n).reshape(1, 1, n, n)
    for cut in range(n + 1):
        a = oracle.partial_attention(q, kk, v, 1.0, 0, cut)
        b = oracle.partial_attention(q, kk, v, 1.0, cut, n)
        o, lse = oracle.merge_partials(np.stack([a[0], b[0]]), np.stack([a[1], b[1]]))
        s_glob, m, l, _ = oracle.two_block_softmax(x, cut)
        assert np.abs(o[0, 0, 0] - s_glob).max() <= 1e-14
        assert abs(lse[0, 0, 0] - (m + np.log(l))) <= 1e-13


@pytest.mark.parametrize("kind", ["unnormalised", "max_not_lse", "equal_weights"])
def test_planted_merge_mistakes_fail_a_pin(kind):
    def bad_merge(o_parts, lse_parts):
        if kind == "unnormalised":
            w = np.exp(lse_parts)
            return (w[..., None] * o_parts).sum(axis=0), np.log(w.sum(axis=0))
        if kind == "max_not_lse":
            lse = lse_parts.max(axis=0)
            w = np.exp(lse_parts - lse)
            return (w[..., None] * o_parts).sum(axis=0), lse
        return o_parts.mean(axis=0), np.log(np.exp(lse_parts).sum(axis=0))
    q, k, v = _random_head(9)
    parts = [oracle.partial_attention(q, k, v, 0.7, a, b) for a, b in ((0, 10), (10, 37))]
    o, lse = bad_merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    o_ref, lse_ref = oracle.standard_attention(q, k, v, 0.7)
    assert np.abs(o - o_ref).max() > 1e-6 or np.abs(lse - lse_ref).max() > 1e-6


# ------------------------------------------------------- standalone softmax

def test_softmax_rows_against_scipy_and_brute_force():
    from scipy.special import logsumexp, softmax
    rng = np.random.default_rng(11)
    x = rng.standard_normal((7, 50)) * 5
    x[2, :] = 3.0                                   # constant row: uniform weights
    x[3, 7] = 80.0                                  # one dominant entry
    y, lse = oracle.softmax_rows(x)
    assert np.abs(y - softmax(x, axis=1)).max() <= 1e-15
    assert np.abs(lse - logsumexp(x, axis=1)).max() <= 1e-13
    assert np.abs(y[2] - 1 / 50).max() <= 1e-16
    assert abs(y[3, 7] - 1.0) <= 1e-15
    assert np.abs(y.sum(axis=1) - 1).max() <= 1e-14
    # 40-digit brute force on one row, no max subtraction
    with decimal.localcontext() as ctx:
        ctx.prec = 40
        row = [D(repr(float(t))) for t in x[0]]
        den = sum(v.exp() for v in row)
        for j, v in enumerate(row):
            assert abs(float(v.exp() / den) - y[0, j]) <= 1e-15 * max(1.0, y[0, j])
        assert abs(float(den.ln()) - lse[0]) <= 1e-13


@pytest.mark.parametrize("n,block", [(1, 1), (17, 1), (17, 4), (1000, 33), (1000, 1000)])
def test_online_row_stats_match_two_pass(n, block):
    rng = np.random.default_rng(n + block)
    x = rng.standard_normal(n) * 10 + np.linspace(0, 30, n)    # maximum moves late
    m, l = oracle.online_row_stats(x, block)
    m2, _, l2, _ = oracle.local_softmax(x)
    assert m == m2
    assert abs(l - l2) <= 1e-13 * l2


# ----------------------------------------------------------------- backward

def _loss_and_grads(q, k, v, do, scale):
    # L = sum(O * dO): its gradient with respect to O is dO
    o, _ = oracle.standard_attention(q, k, v, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_against_central_differences(seed):
    rng = np.random.default_rng(seed)
    B, H, N, d = 1, 2, 6, 4
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    scale = 0.6
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = dict(q=q, k=k, v=v)
            args_m = dict(q=q, k=k, v=v)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss_and_grads(args_p["q"], args_p["k"], args_p["v"], do, scale)
                        - _loss_and_grads(args_m["q"], args_m["k"], args_m["v"], do, scale)) / (2 * h)
        assert np.abs(num - g).max() <= 1e-7 * max(1.0, np.abs(g).max()), name


def test_backward_against_autograd():
    rng = np.random.default_rng(7)
    B, H, N, d = 2, 3, 33, 16
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    scale = 0.25
    dq, dk, dv, D = oracle.attention_backward(q, k, v, do, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.softmax(scale * tq @ tk.transpose(-1, -2), dim=-1) @ tv
    o.backward(torch.tensor(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(mine - ref.numpy()).max() <= 1e-12 * max(1.0, np.abs(mine).max())
    assert np.abs(D - (o.detach().numpy() * do).sum(-1)).max() <= 1e-12


def test_backward_closed_forms():
    rng = np.random.default_rng(8)
    B, H, N, d = 1, 1, 20, 8
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    zero = oracle.attention_backward(q, k, v, np.zeros_like(q), 0.5)
    assert all(np.all(g == 0) for g in zero[:3])
    do = rng.standard_normal((B, H, N, d))
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.5)
    # shifting every key by one vector leaves the output unchanged, so the
    # key gradients sum to zero over the keys; the same holds for queries'
    # effect on dV: dV rows sum to the column sums of dO (P rows sum to 1)
    assert np.abs(dk.sum(axis=2)).max() <= 1e-12
    assert np.abs(dv.sum(axis=2) - do.sum(axis=2)).max() <= 1e-12
    # identical value rows: the output does not depend on Q or K
    vc = np.broadcast_to(rng.standard_normal(d), v.shape).copy()
    dq2, dk2, _, _ = oracle.attention_backward(q, k, vc, do, 0.5)
    assert np.abs(dq2).max() <= 1e-12 and np.abs(dk2).max() <= 1e-12


@pytest.mark.parametrize("kind", ["no_D", "no_scale", "transposed_ds"])
def test_planted_backward_mistakes_fail_a_pin(kind):
    import oracle.backward as ob
    rng = np.random.default_rng(9)
    q, k, v, do = (rng.standard_normal((1, 1, 12, 4)) for _ in range(4))
    good = ob.attention_backward(q, k, v, do, 0.5)
    s = 0.5 * (q[0, 0] @ k[0, 0].T)
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    dp = do[0, 0] @ v[0, 0].T
    D = (do[0, 0] * (p @ v[0, 0])).sum(1)
    if kind == "no_D":
        dq = 0.5 * (p * dp) @ k[0, 0]
    elif kind == "no_scale":
        dq = (p * (dp - D[:, None])) @ k[0, 0]
    else:
        dq = 0.5 * (p * (dp - D[:, None])).T @ k[0, 0]
    assert np.abs(dq - good[0][0, 0]).max() > 1e-6


# ------------------------------------------------------------- FP8 inputs

def test_decode_e4m3_every_code():
    # library conversion of all 256 codes (torch's float8_e4m3fn)
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all()


def test_decode_e4m3_format_landmarks():
    # values fixed by the format: bias 7, 3 mantissa bits, no infinities
    d = lambda c: float(oracle.decode_e4m3(np.array([c], dtype=np.uint8))[0])  # noqa: E731
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0          # largest finite
    assert d(0x08) == 2.0 ** -6                             # smallest normal
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9  # subnormals
    assert d(0x38) == 1.0 and d(0x3C) == 1.5 and d(0x40) == 2.0
    assert d(0x00) == 0.0 and d(0x80) == 0.0 and np.signbit(d(0x80))
    pos = oracle.decode_e4m3(np.arange(0x7F, dtype=np.uint8))
    assert (np.diff(pos) > 0).all()
    # spacing within binade e (codes 8e .. 8e+7, e >= 1) is 2^(e - 10)
    for e in range(1, 16):
        hi = min(8 * e + 8, 0x7F)
        assert (np.diff(pos[8 * e:hi]) == 2.0 ** (e - 10)).all()


def _fp8_tiny(seed, B=1, H=2, N=9, d=4):
    rng = np.random.default_rng(seed)
    codes = [rng.integers(0, 256, size=(B, H, N, d)).astype(np.uint8) for _ in range(3)]
    for c in codes:
        c[(c & 0x7F) == 0x7F] = 0x3A        # finite codes only
    return codes


def test_fp8_attention_against_brute_force():
    # plain Python loops over values decoded by torch's conversion
    q8, k8, v8 = _fp8_tiny(3)
    scale, sq, sk, sv = 0.375, 0.0625, 0.5, 3.0
    o, lse = oracle.fp8_attention(q8, k8, v8, scale, sq, sk, sv)
    dec = lambda c: torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).double().numpy()  # noqa: E731
    q, k, v = sq * dec(q8), sk * dec(k8), sv * dec(v8)
    B, H, N, d = q.shape
    for b in range(B):
        for h in range(H):
            for i in range(N):
                s = [scale * sum(q[b, h, i, c] * k[b, h, j, c] for c in range(d))
                     for j in range(N)]
                m = max(s)
                f = [math.exp(x - m) for x in s]
                l_ = sum(f)
                for c in range(d):
                    ref = sum(f[j] * v[b, h, j, c] for j in range(N)) / l_
                    assert abs(o[b, h, i, c] - ref) <= 1e-12 * (1 + abs(ref))
                assert abs(lse[b, h, i] - (m + math.log(l_))) <= 1e-12 * (1 + abs(m))


def test_fp8_attention_closed_forms_and_scale_roles():
    q8, k8, v8 = _fp8_tiny(4, N=11, d=8)
    # every key row equal: uniform weights, O = v_scale * mean of the V values,
    # LSE = the common score + ln N
    k_eq = np.broadcast_to(k8[:, :, :1], k8.shape).copy()
    sq, sk, sv, scale = 0.25, 2.0, 0.125, 0.5
    o, lse = oracle.fp8_attention(q8, k_eq, v8, scale, sq, sk, sv)
    vals = oracle.decode_e4m3(v8) * sv
    assert np.abs(o - vals.mean(axis=2, keepdims=True)).max() <= 1e-12 * np.abs(vals).max()
    s0 = scale * sq * sk * (oracle.decode_e4m3(q8) * oracle.decode_e4m3(k_eq[:, :, :1])).sum(-1)
    assert np.abs(lse - (s0 + math.log(11))).max() <= 1e-12 * (1 + np.abs(s0).max())
    # only scale * q_scale * k_scale enters the scores; O is linear in v_scale
    o1, l1 = oracle.fp8_attention(q8, k8, v8, 0.5, 0.25, 2.0, 1.0)
    o2, l2 = oracle.fp8_attention(q8, k8, v8, 0.125, 4.0, 0.5, 3.0)
    assert np.abs(o2 - 3.0 * o1).max() <= 1e-12 * (1 + np.abs(o1).max())
    assert np.abs(l2 - l1).max() <= 1e-12 * (1 + np.abs(l1).max())


@pytest.mark.parametrize("kind", ["bias8", "subnormal_exp", "mantissa16", "no_sign",
                                  "v_scale_on_q"])
def test_planted_fp8_mistakes_fail_a_pin(kind, monkeypatch):
    import oracle.fp8 as of
    real = of.decode_e4m3

    def mutant_decode(codes):
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        sign, e, m = (c >> 7) & 1, (c >> 3) & 15, (c & 7).astype(np.float64)
        bias = 8 if kind == "bias8" else 7
        div = 16.0 if kind == "mantissa16" else 8.0
        sub_e = -7 if kind == "subnormal_exp" else -6
        mag = np.where(e == 0, np.ldexp(m / div, sub_e),
                       np.ldexp(1.0 + m / div, (e - bias).astype(np.int32)))
        mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
        return mag if kind == "no_sign" else np.where(sign == 1, -mag, mag)

    if kind == "v_scale_on_q":
        def mutant_values(q8, k8, v8, q_scale, k_scale, v_scale):
            return (v_scale * real(q8), k_scale * real(k8), q_scale * real(v8))
        monkeypatch.setattr(of, "fp8_values", mutant_values)
    else:
        monkeypatch.setattr(of, "decode_e4m3", mutant_decode)
        monkeypatch.setattr(oracle, "decode_e4m3", mutant_decode)
    pins = (test_decode_e4m3_every_code, test_decode_e4m3_format_landmarks,
            test_fp8_attention_against_brute_force,
            test_fp8_attention_closed_forms_and_scale_roles)
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"mutant {kind!r} passed every pin"


# -------------------------------------------- FP8 inputs, selected query rows

def _fp8_rows_brute(q8, k8, v8, scale, sq, sk, sv, rows):
    """Plain loops over the selected rows of every head: values decoded by
    torch's float8_e4m3fn conversion, scales rounded to fp32 (what the GPU
    receives) and widened."""
    dec = lambda c: torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).double().numpy()  # noqa: E731
    f32 = lambda x: float(np.float32(x))  # noqa: E731
    q, k, v = f32(sq) * dec(q8), f32(sk) * dec(k8), f32(sv) * dec(v8)
    B, H, N, d = q.shape
    o = np.empty((B, H, len(rows), v.shape[3]))
    lse = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            for r, i in enumerate(rows):
                s = [f32(scale) * sum(q[b, h, i, c] * k[b, h, j, c] for c in range(d))
                     for j in range(N)]
                m = max(s)
                f = [math.exp(x - m) for x in s]
                l_ = sum(f)
                for c in range(v.shape[3]):
                    o[b, h, r, c] = sum(f[j] * v[b, h, j, c] for j in range(N)) / l_
                lse[b, h, r] = m + math.log(l_)
    return o, lse


def fp8_rows_pin_holds(rows_fn):
    """The selected-rows form of the FP8 oracle against (1) plain loops on
    those rows, with tensor and softmax scales that fp32 does not hold
    exactly (so a scale used without its fp32 rounding moves the result by
    ~1e-8 relative, far above the 1e-12 bar), and (2) the full form on the
    same rows, for row lists that are unsorted, repeated and not a prefix."""
    q8, k8, v8 = _fp8_tiny(11, B=2, H=2, N=13, d=6)
    scale, sq, sk, sv = 0.1, 1.0 / 3.0, 0.7, 2.0 / 7.0
    for rows in ([12, 0, 5], [3, 3, 9, 1], [7]):
        rows = np.array(rows)
        o, lse = rows_fn(q8, k8, v8, scale, sq, sk, sv, rows)
        bo, bl = _fp8_rows_brute(q8, k8, v8, scale, sq, sk, sv, rows)
        assert o.shape == bo.shape and lse.shape == bl.shape
        assert np.abs(o - bo).max() <= 1e-12 * (1 + np.abs(bo).max())
        assert np.abs(lse - bl).max() <= 1e-12 * (1 + np.abs(bl).max())
        fo, fl = oracle.fp8_attention(q8, k8, v8, scale, sq, sk, sv)
        assert np.abs(o - fo[:, :, rows]).max() <= 1e-13 * (1 + np.abs(fo).max())
        assert np.abs(lse - fl[:, :, rows]).max() <= 1e-13 * (1 + np.abs(fl).max())
    return True


def test_fp8_attention_rows_pinned():
    assert fp8_rows_pin_holds(oracle.fp8_attention_rows)


@pytest.mark.parametrize("kind", ["rows_ignored", "scale_not_widened_from_fp32",
                                  "tensor_scales_not_widened", "rows_of_first_head"])
def test_planted_fp8_rows_mistakes_fail_the_pin(kind):
    import oracle.fp8 as of

    def mutant(q8, k8, v8, scale, q_scale, k_scale, v_scale, rows):
        if kind == "tensor_scales_not_widened":
            q, k, v = (q_scale * of.decode_e4m3(q8), k_scale * of.decode_e4m3(k8),
                       v_scale * of.decode_e4m3(v8))
        else:
            q, k, v = of.fp8_values(q8, k8, v8, q_scale, k_scale, v_scale)
        s = float(np.float32(scale)) if kind != "scale_not_widened_from_fp32" else scale
        if kind == "rows_ignored":
            rows = np.arange(len(rows))
        o, lse = oracle.standard_attention_rows(q, k, v, s, rows)
        if kind == "rows_of_first_head":
            o, lse = o.copy(), lse.copy()
            o[:, 1:], lse[:, 1:] = o[:, :1], lse[:, :1]
        return o, lse

    with pytest.raises(AssertionError):
        fp8_rows_pin_holds(mutant)
