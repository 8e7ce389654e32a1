"""The scaled e2m1 -> bf16 conversion (v_cvt_scalef32_pk_bf16_fp4) measured on
the device with fp32 scales that are not powers of two.

The instruction applies only the power of two of the scale's exponent field:
e2m1(code) * 2^(E - 127), E being the fp32 exponent field, the mantissa
ignored.  The MXFP4 dequantisation of the grouped GEMMs relies on this form
(it passes the e8m0 byte as that exponent field); an NVFP4 e4m3 block scale,
which has mantissa bits, therefore cannot go through the conversion and is
multiplied in fp32 instead (e2m1 times e4m3 is exact there and in bf16).
The check runs every e2m1 code against every positive normal-as-fp32 e4m3
value; the probe runs one thread per element and every access is in bounds.
"""
import ctypes

import numpy as np
import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float64)


def e2m1_value(code):
    v = E2M1[code & 7]
    return -v if code & 8 else v


def e4m3_value(b):
    """OCP e4m3 (FN): bias 7, exponent field 0 subnormal, S.1111.111 NaN."""
    s = -1.0 if b & 0x80 else 1.0
    E, m = (b >> 3) & 15, b & 7
    if E == 15 and m == 7:
        return None
    if E == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (E - 7)


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_probe
    torch.cuda.set_device(0)
    return gpu_probe.lib()


def _run(probe, words, scales):
    n = len(words)
    w = torch.from_numpy(np.asarray(words, np.uint32).view(np.int32)).to("cuda")
    s = torch.from_numpy(np.asarray(scales, np.float32)).to("cuda")
    out = torch.empty((n, 8), dtype=torch.int16, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert probe.probe_cvt_fp4_bf16(w.data_ptr(), s.data_ptr(), out.data_ptr(), n, st) == 0
    torch.cuda.synchronize()
    bits = out.cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def test_scale_is_its_exponent_only(probe):
    # two words hold the 16 codes: element j of word w is code 8 w + j
    packed = [sum(((8 * w + j) & 15) << (4 * j) for j in range(8)) for w in range(2)]
    scales = [e4m3_value(b) for b in range(1, 0x7F)]          # positive, nonzero, finite
    words = [packed[w] for v in scales for w in range(2)]
    sc = [v for v in scales for w in range(2)]
    got = _run(probe, words, sc)
    pow2 = lambda v: 2.0 ** np.floor(np.log2(v))
    want = np.array([[e2m1_value(8 * w + j) * pow2(v) for j in range(8)] for v in scales for w in range(2)])
    exact = np.array([[e2m1_value(8 * w + j) * v for j in range(8)] for v in scales for w in range(2)])
    bad = np.nonzero(got != want)
    say(f"  {want.size} conversions: {int(np.sum(got == want))} equal code * 2^exponent(scale), "
        f"{int(np.sum(got == exact))} equal code * scale")
    assert len(bad[0]) == 0, [(sc[i], 8 * (i % 2) + j, got[i, j], want[i, j])
                              for i, j in zip(*bad)][:8]
