"""v_mfma_f32_4x4x4_16b_bf16 measured on the device: its operand layout and
that it sums exact products.

The instruction runs 16 independent 4 x 4 x 4 products per wave.  The layout
the decode-batch streams rely on: lane 4 b + i holds row i of block b's A (its
4 K values, in order), lane 4 b + j holds column j of block b's B, and lane
4 b + j's accumulator register i is block b's output (i, j).  The inputs are
small integers (every sum exact in fp32), so each output names one (b, i, j);
the test also reports which of the other plausible layouts the device
matches, should it not match this one.  One wave per call; every access is in
bounds.
"""
import itertools

import numpy as np
import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_probe
    torch.cuda.set_device(0)
    return gpu_probe.lib()


def _bf16_bits(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _run(probe, A, B, C):
    """A, B: [n][64][4] float32 (bf16-exact), C: [n][64][4] -> D [n][64][4]."""
    n = A.shape[0]
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    a, b = dev(_bf16_bits(A).view(np.int16)), dev(_bf16_bits(B).view(np.int16))
    c = dev(C.astype(np.float32))
    d = torch.empty((n, 64, 4), dtype=torch.float32, device="cuda")
    import ctypes
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert probe.probe_mfma_4x4_bf16(a.data_ptr(), b.data_ptr(), c.data_ptr(), d.data_ptr(), n, st) == 0
    torch.cuda.synchronize()
    return d.cpu().numpy().astype(np.float64)


# lane of (block, index) under two placements
PLACE = {"4b+x": lambda b, x: 4 * b + x, "b+16x": lambda b, x: b + 16 * x}


def _expect(A, B, C, pa, pb, pd):
    """D under placements pa (A rows), pb (B columns), pd (D: lane by column or
    by row, register the other)."""
    n = A.shape[0]
    D = np.zeros((n, 64, 4))
    for c, b, i, j in itertools.product(range(n), range(16), range(4), range(4)):
        la, lb = PLACE[pa](b, i), PLACE[pb](b, j)
        s = float(np.dot(A[c, la].astype(np.float64), B[c, lb].astype(np.float64)))
        if pd == "lane=col":
            ld, r = 4 * b + j, i
        else:
            ld, r = 4 * b + i, j
        D[c, ld, r] = s + C[c, ld, r]
    return D


def test_layout_and_exact_sums(probe):
    rng = np.random.default_rng(41)
    n = 8
    A = rng.integers(-8, 9, (n, 64, 4)).astype(np.float32)
    B = rng.integers(-8, 9, (n, 64, 4)).astype(np.float32)
    C = rng.integers(-64, 65, (n, 64, 4)).astype(np.float32)
    got = _run(probe, A, B, C)
    found = [(pa, pb, pd) for pa in PLACE for pb in PLACE for pd in ("lane=col", "lane=row")
             if np.array_equal(got, _expect(A, B, C, pa, pb, pd))]
    say(f"  layouts matching the device: {found}")
    assert ("4b+x", "4b+x", "lane=col") in found, found


def test_products_exact_in_fp32(probe):
    # bf16 operands with full 8-bit significands: each product is exact in
    # fp32 and four of them plus the accumulator stay well inside 24 bits
    rng = np.random.default_rng(42)
    n = 16
    A = (rng.integers(128, 256, (n, 64, 4)) * rng.choice([-1, 1], (n, 64, 4))).astype(np.float32) / 128
    B = (rng.integers(128, 256, (n, 64, 4)) * rng.choice([-1, 1], (n, 64, 4))).astype(np.float32) / 64
    C = np.zeros((n, 64, 4), np.float32)
    got = _run(probe, A, B, C)
    want = _expect(A, B, C, "4b+x", "4b+x", "lane=col")
    assert np.array_equal(got, want), np.max(np.abs(got - want))
