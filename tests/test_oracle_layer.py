"""Pins for the oracle's expert FFN, combine and whole layer.

Independent references: 60-digit mpmath evaluation of the expert FFN on small
non-square shapes, the hand-computed layers of tests/golden/hand_layers.txt, and
metamorphic relations that hold exactly (power-of-two scaling, identical
experts, relabelled experts).
"""
import math

import mpmath
import numpy as np
import pytest

import synth
from exact import bits_of_f32, read_golden


def _mp_expert(Wg, Wu, Wd, x):
    mpmath.mp.dps = 60
    I, H = Wg.shape
    xs = [mpmath.mpf(float(v)) for v in x]
    h = []
    for j in range(I):
        g = mpmath.fsum(mpmath.mpf(float(Wg[j, i])) * xs[i] for i in range(H))
        u = mpmath.fsum(mpmath.mpf(float(Wu[j, i])) * xs[i] for i in range(H))
        h.append(g / (1 + mpmath.exp(-g)) * u)
    return [mpmath.fsum(mpmath.mpf(float(Wd[o, j])) * h[j] for j in range(I)) for o in range(H)]


def test_expert_ffn_vs_mpmath_nonsquare(orc):
    rng = np.random.default_rng(1)
    H, I = 48, 20                                       # H != I catches transposes
    Wg = rng.standard_normal((I, H)).astype(np.float32)
    Wu = rng.standard_normal((I, H)).astype(np.float32)
    Wd = rng.standard_normal((H, I)).astype(np.float32)
    x = rng.standard_normal(H).astype(np.float32)
    y = orc.expert_ffn(Wg, Wu, Wd, x)
    ref = np.array([float(v) for v in _mp_expert(Wg, Wu, Wd, x)])
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    # gate and up are not interchangeable: silu(g)*u != silu(u)*g
    y_swapped = orc.expert_ffn(Wu, Wg, Wd, x)
    assert np.max(np.abs(y_swapped - ref)) > 1e-3 * np.max(np.abs(ref))


def test_expert_hidden_matches_ffn_first_half(orc):
    rng = np.random.default_rng(2)
    H, I = 32, 16
    Wg = rng.standard_normal((I, H)).astype(np.float32)
    Wu = rng.standard_normal((I, H)).astype(np.float32)
    x = rng.standard_normal(H).astype(np.float32)
    h = orc.expert_hidden(Wg, Wu, x)
    eye = np.eye(I, dtype=np.float32)
    Wd = np.zeros((H, I), np.float32)
    Wd[:I, :I] = eye                                     # y[o] = h[o] for o < I
    y = orc.expert_ffn(Wg, Wu, Wd, x)
    assert np.array_equal(y[:I], h) and np.all(y[I:] == 0)


def test_combine_vs_fsum(orc):
    rng = np.random.default_rng(4)
    w = rng.random(5)
    ys = rng.standard_normal((5, 40))
    out = orc.combine(w, ys)
    for o in range(40):
        assert abs(out[o] - math.fsum(w[s] * ys[s, o] for s in range(5))) < 1e-14


def _pack(c):
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def _hand_layer(orc, k, expert1_code):
    H = I = 32
    Wr = np.zeros((2, H), np.float32)
    Wr[0, 0] = 1.0
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0
    L, idx, w = orc.route(x, Wr, k)
    ws = []
    for e in range(2):
        code = 2 if e == 0 else expert1_code
        mats = [orc.dequant(1, _pack(np.full(s, code, np.uint8)), np.full((s[0], s[1] // 32), 127, np.uint8))
                for s in [(I, H), (I, H), (H, I)]]
        ws.append(mats)
    ys = np.stack([orc.expert_ffn(*ws[e], x[0]) for e in idx[0]])
    return idx[0], w[0], orc.combine(w[0], ys)


def test_hand_layers(orc):
    g = {k: v for k, v in read_golden("hand_layers.txt")}
    idx, w, out = _hand_layer(orc, 1, 0)
    assert idx.tolist() == [0] and w.tolist() == [1.0]
    closed = 32 * math.e / (1 + math.e)
    assert abs(out[0] - float(g["L1_out"])) < 1e-13 and abs(out[0] - closed) < 1e-13
    assert np.all(out == out[0])
    assert bits_of_f32(np.float32(out[0])) == int(g["L1_out_f32_bits"], 16)
    idx, w, out = _hand_layer(orc, 2, 2)
    assert idx.tolist() == [0, 1]
    s1, s0 = 1 / (1 + math.exp(-1)), 0.5
    assert abs(w[0] - s1 / (s1 + s0)) < 1e-15 and abs(w[1] - s0 / (s1 + s0)) < 1e-15
    assert abs(out[0] - float(g["L2_out"])) < 1e-13


# ---------------------------------------------------------------------------
# Whole-layer metamorphic relations on seeded synthetic banks
# ---------------------------------------------------------------------------
def _layer_with(orc, spec, Wr, x, k, edit=None, relabel=None):
    def weights(e):
        src = relabel[e] if relabel is not None else e
        t = synth.expert_tensors(spec, src)
        if edit:
            edit(t)
        g = t["globals"]
        return (orc.dequant(spec.fmt, t["gate_codes"], t["gate_scales"], g[0]),
                orc.dequant(spec.fmt, t["up_codes"], t["up_scales"], g[1]),
                orc.dequant(spec.fmt, t["down_codes"], t["down_scales"], g[2]))
    L, idx, w = orc.route(x, Wr, k)
    out = np.empty((x.shape[0], spec.hidden))
    for t in range(x.shape[0]):
        ys = np.stack([orc.expert_ffn(*weights(int(e)), x[t]) for e in idx[t]])
        out[t] = orc.combine(w[t], ys)
    return idx, out


@pytest.mark.parametrize("fmt", [synth.FMT_MX, synth.FMT_NV])
def test_layer_matches_helper_and_down_scale_doubling(orc, fmt):
    wl = synth.WORKLOADS["tiny"].with_(fmt=fmt)
    spec = wl.bank(0)
    Wr, x = synth.layer_inputs(wl, 0)
    res = orc.layer(spec, Wr, x, wl.k)
    idx, out = _layer_with(orc, spec, Wr, x, wl.k)
    assert np.array_equal(idx, res["idx"]) and np.array_equal(out, res["out"])

    def double_down(t):
        if fmt == synth.FMT_MX:
            t["down_scales"] = (t["down_scales"] + 1).astype(np.uint8)
        else:
            t["globals"] = t["globals"] * np.float32([1, 1, 2])   # down only
    _, out2 = _layer_with(orc, spec, Wr, x, wl.k, edit=double_down)
    assert np.array_equal(out2, 2 * out)


def test_layer_identical_experts_routing_independent(orc):
    wl = synth.WORKLOADS["tiny"]
    spec = wl.bank(0)
    Wr, x = synth.layer_inputs(wl, 0)
    _, out_a = _layer_with(orc, spec, Wr, x, wl.k, relabel=[3] * wl.E)
    _, out_b = _layer_with(orc, spec, Wr[::-1].copy(), x, wl.k, relabel=[3] * wl.E)
    assert np.max(np.abs(out_a - out_b)) <= 1e-12 * np.max(np.abs(out_a))
    y = orc.expert_ffn(*orc.expert_weights(spec, 3), x[0])
    assert np.max(np.abs(out_a[0] - y)) <= 1e-12 * np.max(np.abs(y))


def test_layer_relabel_experts(orc):
    wl = synth.WORKLOADS["tiny"]
    spec = wl.bank(0)
    Wr, x = synth.layer_inputs(wl, 0)
    perm = np.random.default_rng(9).permutation(wl.E)
    idx, out = _layer_with(orc, spec, Wr, x, wl.k)
    # expert e of the relabelled layer is expert perm[e] of the original
    idx2, out2 = _layer_with(orc, spec, Wr[perm], x, wl.k, relabel=perm)
    assert np.array_equal(perm[idx2], idx)
    assert np.array_equal(out2, out)
