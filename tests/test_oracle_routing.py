"""Pins for the oracle's router, selection and routing weights.

Independent references: exact rational dot products (with Higham's bound for the
fp64 sum), brute force over all k-subsets, Python's own sort, closed forms.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest


def _brute_topk(vals, k):
    """The k-subset whose (value desc, index asc) key list is lexicographically
    largest, listed in that order (NaN ranks below every number)."""
    def key(e):
        v = vals[e]
        return (0 if math.isnan(v) else 1, -math.inf if math.isnan(v) else v, -e)
    best = None
    for sub in itertools.combinations(range(len(vals)), k):
        ks = sorted((key(e) for e in sub), reverse=True)
        if best is None or ks > best[0]:
            best = (ks, sub)
    return [-kk[2] for kk in best[0]]


@pytest.mark.parametrize("seed", range(30))
def test_topk_brute_force_with_ties(orc, seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 10))
    k = int(rng.integers(1, E + 1))
    vals = rng.integers(-3, 4, E).astype(np.float64)   # many ties
    got = orc.topk(vals, k)[0].tolist()
    assert got == _brute_topk(vals.tolist(), k)
    assert got == sorted(range(E), key=lambda e: (-vals[e], e))[:k]


def test_topk_adversarial(orc):
    assert orc.topk(np.zeros(8), 3)[0].tolist() == [0, 1, 2]            # all equal
    assert orc.topk(np.array([0.0, -0.0, 0.0]), 2)[0].tolist() == [0, 1]  # -0 == +0
    v = np.array([-0.0, 0.0, -1.0])
    assert orc.topk(v, 1)[0].tolist() == [0]
    v = np.array([1.0, 5.0, 2.0, 3.0])
    assert orc.topk(v, 4)[0].tolist() == [1, 3, 2, 0]                     # k == E
    assert orc.topk(v, 1)[0].tolist() == [1]
    v = np.array([np.nan, -np.inf, 2.0, np.nan, 7.0])
    assert orc.topk(v, 5)[0].tolist() == [4, 2, 1, 0, 3]                 # NaN last
    assert orc.topk(v, 3)[0].tolist() == _brute_topk(v.tolist(), 3)


def test_topk_f32_selects_on_f32_values(orc):
    # two values that differ in fp64 but round to the same fp32 tie -> index order
    a = np.array([1.0 + 2.0 ** -30, 1.0], np.float64)
    assert orc.topk(a, 1)[0].tolist() == [0]
    assert orc.topk(a[::-1].copy(), 1)[0].tolist() == [1]
    assert orc.topk(a[::-1].astype(np.float32), 1)[0].tolist() == [0]   # fp32 tie
    b = np.array([1.0, 1.0 + 2.0 ** -30], np.float64)
    assert orc.topk(b, 1)[0].tolist() == [1]
    assert orc.topk(b.astype(np.float32), 1)[0].tolist() == [0]


def test_topk_large_against_sort(orc):
    rng = np.random.default_rng(7)
    for E, k in [(448, 16), (448, 8), (896, 16), (1024, 32)]:
        vals = rng.standard_normal(E)
        vals[rng.integers(0, E, 20)] = vals[0]                            # plant ties
        got = orc.topk(vals, k)[0].tolist()
        assert got == sorted(range(E), key=lambda e: (-vals[e], e))[:k]


def test_router_exact_within_higham(orc):
    """fp64 sequential dot vs the exact rational value: |err| <= gamma_H sum|x w|."""
    rng = np.random.default_rng(11)
    C, E, H = 3, 5, 96
    x = rng.standard_normal((C, H)).astype(np.float32)
    W = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    L = orc.router_logits(x, W)
    u = 2.0 ** -53
    gam = H * u / (1 - H * u)
    for t in range(C):
        for e in range(E):
            exact = sum(Fraction(float(x[t, h])) * Fraction(float(W[e, h])) for h in range(H))
            bound = gam * sum(abs(float(x[t, h]) * float(W[e, h])) for h in range(H))
            assert abs(Fraction(L[t, e]) - exact) <= Fraction(bound)
    # orientation: logits[t][e] uses row e of W_r (not a transposed read)
    W2 = np.zeros((E, H), np.float32)
    W2[3, 0] = 2.0
    x2 = np.zeros((1, H), np.float32)
    x2[0, 0] = 1.5
    assert orc.router_logits(x2, W2)[0].tolist() == [0, 0, 0, 3.0, 0]


def test_route_weights_invariants(orc):
    rng = np.random.default_rng(3)
    for k in [1, 2, 8, 16]:
        l = rng.standard_normal(k) * 3
        w = orc.route_weights(l)
        assert abs(math.fsum(w) - 1.0) <= 4 * 2.0 ** -53
        assert np.all(w > 0)
        # larger logit -> larger weight (sigmoid is increasing)
        order = np.argsort(-l, kind="stable")
        assert np.all(np.diff(w[order]) <= 0)
    assert orc.route_weights(np.array([0.37])).tolist() == [1.0]
    w = orc.route_weights(np.full(4, 1.25))
    assert np.all(w == 0.25)


def test_route_weights_closed_form(orc):
    """sigma(ln a) = a / (1 + a): logits (ln 3, 0) give sigmas (3/4, 1/2), so
    w = (3/5, 2/5)."""
    w = orc.route_weights(np.array([math.log(3.0), 0.0]))
    assert abs(w[0] - 0.6) < 1e-15 and abs(w[1] - 0.4) < 1e-15


def test_silu_closed_forms(orc):
    assert orc.silu(0.0) == 0.0
    assert abs(orc.silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15   # sigma(ln 3) = 3/4
    for z in [0.3, 1.7, 5.0, 11.0]:
        assert abs((orc.silu(z) - orc.silu(-z)) - z) < 4e-15 * max(1, z)  # silu(z)-silu(-z)=z
    assert orc.silu(60.0) == 60.0                    # -> z for large z
    assert 0 > orc.silu(-60.0) > -1e-20               # -> -0 for very negative z


def test_route_end_to_end_small(orc):
    rng = np.random.default_rng(21)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    W = (rng.standard_normal((10, 64)) * 0.02).astype(np.float32)
    L, idx, w = orc.route(x, W, 3)
    for t in range(4):
        assert idx[t].tolist() == _brute_topk(L[t].tolist(), 3)
        assert abs(math.fsum(w[t]) - 1) < 1e-15
