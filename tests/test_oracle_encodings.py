"""Pins for the oracle's element encodings and dequantisation.

Independent references: the OCP value list (golden file), torch's own
float8_e8m0fnu / float8_e4m3fn conversions, and exact rational products rounded
to fp32 with integer arithmetic (tests/exact.py).
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

from exact import bits_of_f32, e2m1_exact, f32_from_bits, read_golden, round_f32


def test_e2m1_matches_ocp_table(orc):
    for c, v in read_golden("e2m1_ocp_values.txt"):
        got = orc.e2m1(int(c, 16))
        want = float(v)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (c, got, want)


def test_e2m1_sign_symmetry_and_monotone(orc):
    mags = [orc.e2m1(c) for c in range(8)]
    assert all(a < b for a, b in zip(mags, mags[1:]))
    for c in range(8):
        assert orc.e2m1(c | 8) == -orc.e2m1(c)
    assert math.copysign(1, orc.e2m1(8)) == -1.0   # negative zero


def test_e8m0_matches_torch(orc):
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).float().numpy()
    for b in range(256):
        got = orc.e8m0(b)
        if b == 255:
            assert math.isnan(got) and math.isnan(t[b])
        else:
            assert np.float32(got) == t[b], b
            assert got == 2.0 ** (b - 127)


def test_e4m3_matches_torch(orc):
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for b in range(256):
        got = orc.e4m3(b)
        if math.isnan(t[b]):
            assert math.isnan(got), b
        else:
            assert np.float32(got) == t[b] and math.copysign(1, got) == math.copysign(1, float(t[b])), b
    assert orc.e4m3(0x7E) == 448.0           # largest finite
    assert math.isnan(orc.e4m3(0x7F)) and math.isnan(orc.e4m3(0xFF))


def _pack(codes):
    codes = np.asarray(codes, np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def test_dequant_mx_exhaustive(orc):
    """Every code against every e8m0 byte (incl. subnormal 0/1, overflow 254,
    NaN 255): one row per scale byte, 32 elements = 16 codes twice."""
    codes = np.tile(np.arange(16, dtype=np.uint8), (256, 2))      # [256][32]
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    got = orc.dequant(1, _pack(codes), scales)
    for b in range(256):
        for j in range(32):
            c = j % 16
            g = got[b, j]
            if b == 255:
                assert np.isnan(g)
                continue
            want = round_f32(e2m1_exact(c) * Fraction(2) ** (b - 127), negative_zero=(c == 8))
            assert bits_of_f32(g) == bits_of_f32(np.float32(want)), (b, c, g, want)


def test_dequant_nv_exhaustive_codes_scales(orc):
    """16 codes x all 127 positive finite e4m3 bytes x seeded fp32 globals;
    exact rational product rounded once to fp32."""
    rng = np.random.default_rng(123)
    gs = (1.0 + rng.integers(0, 2 ** 23, 40) * 2.0 ** -23).astype(np.float32)
    gs = np.concatenate([gs, np.float32([1.0, 1.1, 1.9999999, 0.75, 3.0e-3])])
    sbytes = np.arange(0, 0x7F, dtype=np.uint8)                   # 0x00..0x7E
    codes = np.tile(np.arange(16, dtype=np.uint8), (len(sbytes), 1))   # [127][16]
    for g in gs:
        got = orc.dequant(2, _pack(np.concatenate([codes, codes], 1)), np.repeat(sbytes[:, None], 2, 1), g)
        gq = Fraction(float(g))
        for i, sb in enumerate(sbytes):
            sq = Fraction(orc.e4m3(int(sb)))
            for c in range(16):
                want = round_f32(e2m1_exact(c) * sq * gq, negative_zero=(c >= 8))
                assert bits_of_f32(got[i, c]) == bits_of_f32(np.float32(want)), (g, sb, c)


def test_nv_worked_example(orc):
    d = {k: v for k, v in read_golden("nv_worked_example.txt")}
    code, sb = int(d["code"], 16), int(d["scale"], 16)
    g = f32_from_bits(int(d["g_bits"], 16))
    packed = np.array([[code | (code << 4)] * 8], np.uint8)        # 16 elements
    got = orc.dequant(2, packed, np.array([[sb]], np.uint8), g)
    assert bits_of_f32(got[0, 0]) == int(d["w_bits"], 16)


def test_mx_nv_reencoding_identical(orc):
    """An MX block scale 2^(b-127) that e4m3 can hold, with g = 1, dequantises
    to the same bits as NV (metamorphic: two encodings of one matrix)."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (64, 64), dtype=np.uint8)          # K = 128
    b = rng.integers(121, 135, (64, 4)).astype(np.uint8)             # 2^-6 .. 2^7
    e4 = ((b.astype(np.int32) - 127 + 7) << 3).astype(np.uint8)     # same power of two
    mx = orc.dequant(1, codes, b)
    nv = orc.dequant(2, codes, np.repeat(e4, 2, axis=1), 1.0)
    assert np.array_equal(mx.view(np.uint32), nv.view(np.uint32))


def test_nibble_order(orc):
    """Element 2i is the low nibble, element 2i+1 the high nibble."""
    packed = np.zeros((1, 16), np.uint8)
    packed[0, 0] = 0x72          # element 0 = code 2 (1.0), element 1 = code 7 (6.0)
    got = orc.dequant(1, packed, np.array([[127]], np.uint8))
    assert got[0, 0] == 1.0 and got[0, 1] == 6.0 and np.all(got[0, 2:] == 0)
