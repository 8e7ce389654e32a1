"""Pins for the oracle's comparison helpers, which every parity assertion and
every routing acceptance goes through: ``rel_l2``, ``max_abs_ratio`` and
``logit_error_bound``.

Independent references: hand-computed norms, exact rational dot products
(``fractions.Fraction``) of fp32 sums taken in known orders, and sums whose
fp32 result is fixed by round-to-nearest-even (Higham, Accuracy and Stability
of Numerical Algorithms, 2nd ed., section 3.1, for the bound's form).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

U = 2.0 ** -24          # unit roundoff of fp32


# ---------------------------------------------------------------------------
# rel_l2 and max_abs_ratio on hand vectors
# ---------------------------------------------------------------------------
def test_rel_l2_hand_values(orc):
    ref = np.array([3.0, 4.0])                                  # ||ref|| = 5
    assert orc.rel_l2(ref, ref) == 0.0
    assert orc.rel_l2(np.array([3.3, 3.6]), ref) == pytest.approx(0.1, rel=1e-12)   # ||d|| = 0.5
    # the denominator is ||ref||, not ||got||: got = 2 ref gives 1, not 1/2
    assert orc.rel_l2(2 * ref, ref) == pytest.approx(1.0, rel=1e-15)
    # a norm, not its square: ||d|| / ||ref|| = 0.5 (the squared ratio would be 0.25)
    assert orc.rel_l2(np.array([1.5, 0.0]), np.array([1.0, 0.0])) == pytest.approx(0.5, rel=1e-15)
    # over the whole tensor, not per row: sqrt(1) / sqrt(2)
    assert orc.rel_l2(np.array([[1.0, 0.0], [0.0, 2.0]]), np.eye(2)) == pytest.approx(
        1 / math.sqrt(2), rel=1e-15)
    # signs count: got = -ref is 2 away
    assert orc.rel_l2(-ref, ref) == pytest.approx(2.0, rel=1e-15)
    # a zero reference: the absolute norm of the difference
    assert orc.rel_l2(np.array([3.0, 4.0]), np.zeros(2)) == pytest.approx(5.0, rel=1e-15)


def test_max_abs_ratio_hand_values(orc):
    ref = np.array([-4.0, 2.0])
    # max|d| = 1 over max|ref| = 4 (a max without abs would take 2 for ref)
    assert orc.max_abs_ratio(np.array([-3.0, 2.5]), ref) == pytest.approx(0.25, rel=1e-15)
    # the largest difference is negative: d = [-1, 0.5], max|d| = 1, not 0.5
    assert orc.max_abs_ratio(np.array([-5.0, 2.5]), ref) == pytest.approx(0.25, rel=1e-15)
    assert orc.max_abs_ratio(ref, ref) == 0.0
    # the reference's own maximum, not the result's: got = 3 ref gives 2, not 2/3
    assert orc.max_abs_ratio(3 * ref, ref) == pytest.approx(2.0, rel=1e-15)
    assert orc.max_abs_ratio(np.array([0.5, -0.25]), np.zeros(2)) == 0.5
    assert orc.max_abs_ratio(np.zeros(0), np.zeros(0)) == 0.0
    # 2-D, the maximum over the whole tensor
    assert orc.max_abs_ratio(np.array([[1.0, 0.0], [0.0, 1.5]]), np.eye(2)) == pytest.approx(0.5)


# ---------------------------------------------------------------------------
# logit_error_bound against exact errors of fp32 sums in known orders
# ---------------------------------------------------------------------------
def _exact_dot(x, w) -> Fraction:
    return sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, w)), Fraction(0))


def _sum_sequential(p):
    """fp32 products, each rounded, added left to right in fp32: the longest
    chain of roundings is len(p) (the first product's rounding and every add)."""
    acc = np.float32(0.0)
    for v in p:
        acc = np.float32(acc + v)
    return acc, len(p)


def _sum_pairwise(p):
    """fp32 pairwise tree over the products: depth ceil(log2 n) adds + 1."""
    vals = list(p)
    depth = 1
    while len(vals) > 1:
        nxt = [np.float32(vals[i] + vals[i + 1]) for i in range(0, len(vals) - 1, 2)]
        if len(vals) % 2:
            nxt.append(vals[-1])
        vals = nxt
        depth += 1
    return vals[0], depth


def _sum_lanes(p, lanes=64):
    """The decode router's order: lane l adds products l, l + lanes, ... in
    sequence, then a butterfly over the lanes (log2 lanes levels)."""
    n = len(p)
    part = []
    for l in range(lanes):
        acc = np.float32(0.0)
        for i in range(l, n, lanes):
            acc = np.float32(acc + p[i])
        part.append(acc)
    per_lane = (n + lanes - 1) // lanes
    s, d = _sum_pairwise(part)
    return s, per_lane + d


@pytest.mark.parametrize("order", [_sum_sequential, _sum_pairwise, _sum_lanes])
@pytest.mark.parametrize("seed", range(4))
def test_logit_bound_holds_for_fp32_sums(orc, order, seed):
    """|fp32 sum - exact| <= bound(depth of that order), for N(0,1) x N(0,0.02)
    products at H = 512, 8 experts."""
    rng = np.random.default_rng(100 + seed)
    H, E = 512, 8
    x = rng.standard_normal((1, H)).astype(np.float32)
    W = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    for e in range(E):
        p = [np.float32(a * b) for a, b in zip(x[0], W[e])]
        s, depth = order(p)
        bound = orc.logit_error_bound(x, W[[e]], depth)[0, 0]
        err = abs(Fraction(float(s)) - _exact_dot(x[0], W[e]))
        assert err <= Fraction(float(bound)), (order.__name__, e, float(err), bound)


def test_logit_bound_tight_on_absorbed_sum(orc):
    """1 + n * 2^-24 summed left to right in fp32: every 2^-24 ties with the
    running 1 and rounds to even (down), so the error is exactly n * 2^-24.
    The bound for depth n + 1 is (n + 1) u (1 + n u) / (1 - (n + 1) u): within
    (n + 1) / n of the error.  A unit roundoff of 2^-25 would put the bound
    below the error; 2^-23 would make it twice as loose."""
    n = 64
    x = np.ones((1, n + 1), np.float32)
    w = np.array([[1.0] + [U] * n], np.float32)
    p = [np.float32(a * b) for a, b in zip(x[0], w[0])]
    s, depth = _sum_sequential(p)
    assert float(s) == 1.0 and depth == n + 1
    err = float(_exact_dot(x[0], w[0]) - Fraction(float(s)))
    assert err == n * U
    bound = float(orc.logit_error_bound(x, w, depth)[0, 0])
    assert err <= bound <= err * (n + 1) / n * 1.001


def test_logit_bound_uses_absolute_products(orc):
    """1 + n * 2^-24 - 1: the fp32 sum is 0, the exact value n * 2^-24.  The
    bound scales with sum |x_h w_h| (about 2), not with |sum x_h w_h| (n u): a
    bound on the signed sum would be far below the error."""
    n = 64
    x = np.ones((1, n + 2), np.float32)
    w = np.array([[1.0] + [U] * n + [-1.0]], np.float32)
    p = [np.float32(a * b) for a, b in zip(x[0], w[0])]
    s, depth = _sum_sequential(p)
    assert float(s) == 0.0
    err = float(_exact_dot(x[0], w[0]))
    assert err == n * U
    bound = float(orc.logit_error_bound(x, w, depth)[0, 0])
    assert err <= bound
    gamma = depth * U / (1 - depth * U)
    assert bound == pytest.approx(gamma * (2 + n * U) + 2.0 ** -149, rel=1e-12)


def test_logit_bound_shape_and_rows(orc):
    """[C][E] output; entry (t, e) uses token t and router row e only."""
    x = np.array([[1.0, -2.0], [0.5, 0.0]], np.float32)
    W = np.array([[3.0, 1.0], [-1.0, 4.0], [0.0, 0.0]], np.float32)
    b = orc.logit_error_bound(x, W, 10)
    g = 10 * U / (1 - 10 * U)
    assert b.shape == (2, 3)
    expect = g * np.array([[5.0, 9.0, 0.0], [1.5, 0.5, 0.0]]) + 2.0 ** -149
    np.testing.assert_allclose(b, expect, rtol=1e-14, atol=0)
