"""The seeded input generators: published SplitMix64 vectors, determinism and
the value ranges the workloads state."""
import numpy as np

import synth


def test_splitmix64_published_vectors():
    # SplitMix64 from state 0: the first outputs of the reference generator
    # (Steele, Lea, Flood 2014; Vigna's splitmix64.c).
    assert [int(v) for v in synth.stream_words(0, 0, 3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_expert_bytes_deterministic_and_distinct():
    spec = synth.BankSpec(synth.FMT_MX, 8, 256, 128, seed=0, layer=0)
    a = synth.expert_tensor_bytes(spec, 3, synth.T_GATE_CODES)
    b = synth.expert_tensor_bytes(spec, 3, synth.T_GATE_CODES)
    c = synth.expert_tensor_bytes(spec, 4, synth.T_GATE_CODES)
    d = synth.expert_tensor_bytes(synth.BankSpec(synth.FMT_MX, 8, 256, 128, 0, 1), 3, 0)
    assert np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)
    assert a.shape == (128, 128)


def test_value_ranges():
    mx = synth.BankSpec(synth.FMT_MX, 4, 512, 256)
    nv = synth.BankSpec(synth.FMT_NV, 4, 512, 256)
    codes = synth.expert_tensor_bytes(mx, 0, synth.T_UP_CODES)
    nib = np.concatenate([codes & 15, codes >> 4]).ravel()
    assert set(np.unique(nib).tolist()) == set(range(16))           # all 16 codes
    s = synth.expert_tensor_bytes(mx, 0, synth.T_DOWN_SCALES)
    assert s.shape == (512, 8) and set(np.unique(s).tolist()) == {123, 124, 125, 126, 127}
    s = synth.expert_tensor_bytes(nv, 0, synth.T_GATE_SCALES)
    assert s.shape == (256, 32) and s.min() >= 0x18 and s.max() <= 0x37
    g = synth.global_scales(nv, 2)
    assert g.dtype == np.float32 and np.all((g >= 1) & (g < 2))
    assert nv.expert_bytes() == 3 * (256 * 256 + 256 * 512 // 16) + 12


def test_expert_bytes_match_pages():
    # K3 NVFP4 expert: 3 matrices of 11,010,048 elements -> 18,579,456 bytes of
    # codes and block scales; the pages quote 18,579,480 per expert, i.e. 24 bytes
    # more than that (six fp32 per-tensor values; three are weight scales here).
    nv = synth.BankSpec(synth.FMT_NV, 896, 7168, 1536)
    assert nv.expert_bytes() - 12 == 18_579_456
    mx = synth.BankSpec(synth.FMT_MX, 448, 3584, 3072)
    assert mx.expert_bytes() == 3 * 5_849_088


def test_zipf_sets_distinct_and_skewed():
    sets = synth.zipf_sets(0, 0, 2048, 896, 16, 1.0)
    assert all(len(set(r)) == 16 for r in sets)
    counts = np.bincount(sets.ravel(), minlength=896)
    assert counts.max() > 1000 and np.median(counts) < 60


def test_bf16_rounding():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e-39], np.float32)
    r = synth.round_to_bf16(v)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 2 ** -7 and r[3] == -2.5
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
