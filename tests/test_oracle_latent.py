"""Pins for the oracle's latent MoE layer (bf16 dense products, the RMS norm
after the routed sum, routed_up, the shared experts).

Independent references: hand-computed norms, exact rational sums for the
dense product, the bf16 bit patterns' defined values, and a layer built from
selection matrices, where the dense products only move values and the result
follows from the already pinned router and expert FFN by a closed form
(a normalised vector has mean square 1; the norm of a sum is not the sum of
the norms).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import synth


def test_bf16_values(orc):
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0x3E20, 0x8000], np.uint16)
    v = orc.bf16_matrix(bits)
    assert v[0] == 1.0 and v[1] == -2.0
    assert v[2] == 2.0 ** -133                    # smallest subnormal: 2^-126 * 2^-7
    assert math.isinf(v[3]) and v[3] > 0
    assert v[4] == 0.15625                        # 1.25 * 2^-3
    assert v[5] == 0.0 and math.copysign(1.0, v[5]) < 0


def test_dense_exact_nonsquare(orc):
    """Against exact rational sums of the bf16 values (decoded here from the
    bit patterns) times the fp32 inputs."""
    g = np.random.default_rng(5)
    N, K, C = 3, 37, 2
    Wb = (g.standard_normal((N, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    x = g.standard_normal((C, K)).astype(np.float32)
    y = orc.dense(Wb, x)
    assert y.shape == (C, N)
    for t in range(C):
        for n in range(N):
            wv = [float(np.array([int(b) << 16], np.uint32).view(np.float32)[0]) for b in Wb[n]]
            terms = [Fraction(wv[i]) * Fraction(float(x[t, i])) for i in range(K)]
            scale = float(sum(abs(v) for v in terms))
            assert abs(y[t, n] - float(sum(terms))) <= 1e-14 * scale


def test_dense_selection_matrix_orientation(orc):
    """W [N][K] with W[n][q(n)] = 1 picks x[q(n)]: a transposed operand would
    fail the shape or the positions."""
    N, K = 5, 8
    W = np.zeros((N, K), np.uint16)
    q = [3, 0, 7, 1, 5]
    for n in range(N):
        W[n, q[n]] = 0x3F80
    x = np.arange(2 * K, dtype=np.float32).reshape(2, K) * 0.5 - 3
    y = orc.dense(W, x)
    assert np.array_equal(y, x[:, q].astype(np.float64))


def test_rms_norm_hand_values(orc):
    # [3, 4]: mean square 12.5, so 3 / sqrt(12.5) and 4 / sqrt(12.5)
    y = orc.rms_norm(np.array([[3.0, 4.0]]), np.ones(2), 0.0)
    assert np.allclose(y, [[0.848528137423857, 1.131370849898476]], rtol=0, atol=1e-15)
    # constant 2 over 4 entries with eps 0.25: 2 / sqrt(4 + 0.25), times gamma
    y = orc.rms_norm(np.full((1, 4), 2.0), np.array([1.0, 2.0, 3.0, -1.0]), 0.25)
    r = 2.0 / math.sqrt(4.25)
    assert np.allclose(y, [[r, 2 * r, 3 * r, -r]], rtol=1e-15, atol=0)
    # zero row with eps > 0 stays zero
    assert np.array_equal(orc.rms_norm(np.zeros((1, 8)), np.ones(8), 1e-6), np.zeros((1, 8)))


def test_rms_norm_properties(orc):
    g = np.random.default_rng(9)
    y = g.standard_normal((3, 64)) * np.array([[1e-3], [1.0], [40.0]])
    gam = np.ones(64)
    n = orc.rms_norm(y, gam, 0.0)
    assert np.allclose(np.mean(n * n, axis=1), 1.0, rtol=1e-14)
    assert np.allclose(orc.rms_norm(7.5 * y, gam, 0.0), n, rtol=1e-13, atol=0)
    assert np.allclose(orc.rms_norm(-y, gam, 0.0), -n, rtol=0, atol=0)
    # rows are independent
    assert np.allclose(orc.rms_norm(y[1:2], gam, 0.0), n[1:2], rtol=0, atol=0)
    # eps shrinks a small row towards y / sqrt(eps)
    small = orc.rms_norm(y[:1], gam, 1.0)
    assert np.allclose(small, y[:1] / np.sqrt(np.mean(y[:1] ** 2) + 1.0), rtol=1e-14)


def _tiny(fmt=synth.FMT_MX):
    return synth.LatentWorkload("tiny_latent", fmt, 8, 2, 64, 32, 64, 2, 32, 3, eps=0.0,
                                gamma_scale=1024.0)


def _selection(N, K, pick):
    W = np.zeros((N, K), np.uint16)
    for n, c in pick:
        W[n, c] = 0x3F80
    return W


@pytest.mark.parametrize("fmt", [synth.FMT_MX, synth.FMT_NV])
def test_latent_layer_selection_matrices(orc, fmt):
    """routed_down and routed_up as selection matrices, gamma 1, eps 0: x_lat is
    x at the picked columns, y_lat the weighted sum of the selected experts'
    FFNs at x_lat (router on the hidden x), the routed part y_lat / rms(y_lat)
    at the picked rows and zero elsewhere (mean square exactly 1, which
    normalising each expert before the sum would miss), plus the two shared
    experts' FFNs at x with weight 1."""
    wl = _tiny(fmt)
    Wr, x, _, _, _ = synth.latent_inputs(wl, 0)
    q = [(3 * j + 1) % wl.H for j in range(wl.L)]
    p = [(5 * j + 2) % wl.H for j in range(wl.L)]
    Wd = _selection(wl.L, wl.H, [(j, q[j]) for j in range(wl.L)])
    Wu = _selection(wl.H, wl.L, [(p[j], j) for j in range(wl.L)])
    gamma = np.ones(wl.L, np.float32)
    r = orc.latent_layer(wl, Wr, x, Wd, Wu, gamma)

    _, idx, w = orc.route(x, Wr, wl.k)
    assert np.array_equal(r["idx"], idx)
    rs, ss = wl.routed_bank(), wl.shared_bank()
    sh = [orc.expert_weights(ss, j) for j in range(wl.n_shared)]
    for t in range(wl.C):
        xl = x[t, q]
        assert np.array_equal(r["xlat"][t], xl.astype(np.float64))
        ylat = sum(w[t, s] * orc.expert_ffn(*orc.expert_weights(rs, int(idx[t, s])), xl)
                   for s in range(wl.k))
        assert np.allclose(r["ylat"][t], ylat, rtol=1e-14, atol=1e-300)
        routed = np.zeros(wl.H)
        routed[p] = ylat / math.sqrt(np.mean(ylat * ylat))
        assert np.allclose(r["routed"][t], routed, rtol=1e-13, atol=1e-15)
        assert abs(np.mean(r["routed"][t][p] ** 2) - 1.0) < 1e-13
        # per-expert normalisation would give a smaller mean square here
        per = sum(w[t, s] * orc.rms_norm(orc.expert_ffn(*orc.expert_weights(rs, int(idx[t, s])), xl),
                                         np.ones(wl.L), 0.0) for s in range(wl.k))
        assert np.mean(per * per) < 1.0 - 1e-3
        shared = orc.expert_ffn(*sh[0], x[t]) + orc.expert_ffn(*sh[1], x[t])
        assert np.allclose(r["shared"][t], shared, rtol=1e-15, atol=0)
        assert np.allclose(r["out"][t], routed + shared, rtol=1e-13, atol=1e-15)


def test_latent_layer_up_zero_gamma_linear(orc):
    """W_up = 0 or gamma = 0 leaves the shared experts alone; doubling gamma or
    W_up doubles the routed part exactly (powers of two)."""
    wl = _tiny().with_(eps=1e-6)
    Wr, x, Wd, Wu, gamma = synth.latent_inputs(wl, 0)
    base = orc.latent_layer(wl, Wr, x, Wd, Wu, gamma)
    zero_up = orc.latent_layer(wl, Wr, x, Wd, np.zeros_like(Wu), gamma)
    zero_g = orc.latent_layer(wl, Wr, x, Wd, Wu, np.zeros_like(gamma))
    assert np.array_equal(zero_up["out"], base["shared"])
    assert np.array_equal(zero_g["out"], base["shared"])
    assert np.abs(base["routed"]).max() > 0.1 * np.abs(base["shared"]).max()
    two_g = orc.latent_layer(wl, Wr, x, Wd, Wu, 2 * gamma)
    assert np.array_equal(two_g["routed"], 2 * base["routed"])
    Wu2 = (Wu.astype(np.uint32) + np.where((Wu & 0x7FFF) != 0, 0x80, 0)).astype(np.uint16)
    two_u = orc.latent_layer(wl, Wr, x, Wd, Wu2, gamma)   # exponent + 1: every entry doubled
    assert np.array_equal(two_u["routed"], 2 * base["routed"])
