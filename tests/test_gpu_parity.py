"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: routing indices and dequantised weights bit-exact; fp32 layer outputs
within rel-L2 <= 2e-5 and max-abs <= 1e-4 * max|ref| of the oracle's fp64
result.  Every case prints its name before it runs.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (assert_close, cached_bank, check_selection, make_bank, route_depth, say,
                      to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_fp4_amd as rf
    rf.lib()
    oracle.build()
    torch.cuda.set_device(0)


def rf():
    import routed_expert_fp4_amd
    return routed_expert_fp4_amd


# ---------------------------------------------------------------------------
# Bank bytes and dequantisation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,experts", [("tiny", [0, 7]), ("w50_k16", [0, 447]),
                                          ("k3_stack", [5])])
def test_device_fill_matches_host(name, experts):
    wl = synth.WORKLOADS[name]
    spec = wl.bank(0)
    say(f"[fill] {name} experts {experts}")
    bank = cached_bank(spec)
    for e in experts:
        for t in range(7):
            n = spec.tensor_bytes(t)
            if n == 0:
                continue
            dev = bank.tensor_view(e, t, n).cpu().numpy()
            host = synth.expert_tensor_bytes(spec, e, t).ravel()
            assert np.array_equal(dev, host), (name, e, t)


def _hand_bank(fmt, H, I, gate_codes, gate_scales, g=1.0):
    """A one-expert bank whose gate matrix is given; other tensors zero."""
    b = rf().Bank(fmt, 1, H, I)
    b.storage.zero_()
    b.tensor_view(0, 0, gate_codes.size).copy_(torch.from_numpy(gate_codes.ravel()))
    b.tensor_view(0, 3, gate_scales.size).copy_(torch.from_numpy(gate_scales.ravel()))
    if fmt == synth.FMT_NV:
        gl = np.array([g, 1.0, 1.0], np.float32).view(np.uint8)
        b.tensor_view(0, 6, 12).copy_(torch.from_numpy(gl))
    return b


def _pack(codes):
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _same_bits(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    nan = np.isnan(a) & np.isnan(b)
    return np.all(nan | (a.view(np.uint32) == b.view(np.uint32)))


def test_dequant_mx_exhaustive():
    """All 16 codes x all 256 e8m0 bytes (subnormal, overflow, NaN included)."""
    say("[dequant] mx exhaustive")
    I, H = 256, 32
    codes = np.tile(np.arange(16, dtype=np.uint8), (I, 2))
    scales = np.arange(256, dtype=np.uint8).reshape(I, 1)
    b = _hand_bank(synth.FMT_MX, H, I, _pack(codes), scales)
    out = torch.empty((I, H), dtype=torch.float32, device="cuda")
    rf().moe_dequant(b, 0, 0, out)
    got = out.cpu().numpy()
    ref = oracle.dequant(synth.FMT_MX, _pack(codes), scales)
    assert _same_bits(got, ref)


@pytest.mark.parametrize("g", [1.0, 1.1, 1.9999999, 0.75, 3.0e-3, 1.3370001])
def test_dequant_nv_exhaustive(g):
    """All 16 codes x all 256 e4m3 bytes (subnormals, NaN) x a per-tensor g."""
    say(f"[dequant] nv exhaustive g={g}")
    I, H = 256, 32
    codes = np.tile(np.arange(16, dtype=np.uint8), (I, 2))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 2, 1)
    b = _hand_bank(synth.FMT_NV, H, I, _pack(codes), scales, g)
    out = torch.empty((I, H), dtype=torch.float32, device="cuda")
    rf().moe_dequant(b, 0, 0, out)
    ref = oracle.dequant(synth.FMT_NV, _pack(codes), scales, np.float32(g))
    assert _same_bits(out.cpu().numpy(), ref)


@pytest.mark.parametrize("name,expert", [("tiny", 3), ("w50_k16", 200), ("k3_stack", 801)])
def test_dequant_bank_matrices(name, expert):
    wl = synth.WORKLOADS[name]
    spec = wl.bank(0)
    say(f"[dequant] {name} expert {expert}")
    bank = cached_bank(spec)
    ref = oracle.expert_weights(spec, expert)
    for m in range(3):
        N, K = ref[m].shape
        out = torch.empty((N, K), dtype=torch.float32, device="cuda")
        rf().moe_dequant(bank, expert, m, out)
        assert _same_bits(out.cpu().numpy(), ref[m]), (name, expert, m)


# ---------------------------------------------------------------------------
# Routing
# ---------------------------------------------------------------------------
def _ws(E, H, I, k, C):
    return rf().Workspace(E, H, I, k, C)


@pytest.mark.parametrize("E,k,C,seed", [(8, 2, 4, 0), (448, 16, 1, 1), (448, 8, 7, 2),
                                        (896, 16, 16, 3), (1024, 32, 3, 4), (5, 5, 2, 5),
                                        (64, 1, 1, 6), (896, 16, 40, 7), (1024, 32, 17, 8)])
def test_route_logits_in_bit_exact(E, k, C, seed):
    """Selection on identical fp32 logits: indices bit-exact with the oracle's
    fp32 selection, including planted ties and signed zeros."""
    say(f"[route logits-in] E={E} k={k} C={C}")
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((C, E)).astype(np.float32)
    L[:, rng.integers(0, E, max(1, E // 8))] = L[0, 0]        # ties
    L[0, : min(E, 4)] = 0.0
    if E > 4:
        L[0, 4] = -0.0
    logits = to_dev(L)
    idx = torch.empty((C, k), dtype=torch.int32, device="cuda")
    w = torch.empty((C, k), dtype=torch.float32, device="cuda")
    rf().moe_route(None, None, logits, C, 32, E, k, idx, w, _ws(E, 32, 32, k, C))
    got = idx.cpu().numpy()
    ref = oracle.topk(L, k)
    assert np.array_equal(got, ref)
    wr = np.stack([oracle.route_weights(L[t, ref[t]].astype(np.float64)) for t in range(C)])
    np.testing.assert_allclose(w.cpu().numpy(), wr, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("C", [3, 20])
def test_route_logits_in_all_equal_and_nan(C):
    """All-equal rows, NaN and -inf logits; C = 20 takes the many-token top-k
    launch (one wave per token), whose candidate gather falls back to
    rounds of the wave maximum when more than 64 entries tie."""
    say(f"[route logits-in] adversarial C={C}")
    E, k = 40, 6
    L = np.zeros((C, E), np.float32)
    L[1] = np.linspace(-1, 1, E, dtype=np.float32)
    L[1, [3, 9]] = np.nan
    L[2] = -np.inf
    L[2, 7] = 0.5
    for t in range(3, C):                      # the three patterns again, shifted
        L[t] = np.roll(L[t % 3], t)
    idx = torch.empty((C, k), dtype=torch.int32, device="cuda")
    w = torch.empty((C, k), dtype=torch.float32, device="cuda")
    rf().moe_route(None, None, to_dev(L), C, 32, E, k, idx, w, _ws(E, 32, 32, k, C))
    got = idx.cpu().numpy()
    assert got[0].tolist() == list(range(k))
    assert np.array_equal(got, oracle.topk(L, k))


@pytest.mark.parametrize("name,C", [("tiny", 4), ("w50_k16", 1), ("w50_k8", 1),
                                    ("w50_c7_k16", 7), ("k3_stack", 1), ("k3_stack", 16),
                                    ("k3_stack_zipf", 1), ("k3_stack", 64), ("k3_prefill", 2048)])
def test_route_end_to_end(name, C):
    """The GPU's fp32 logits within the certified bound of the oracle's fp64
    logits for every token and expert (the split-K router up to 16 tokens,
    the matrix-core router above), and the selection equal to the oracle's
    up to certified near-ties (none under steered routing)."""
    wl = synth.WORKLOADS[name]
    say(f"[route e2e] {name} C={C}")
    Wr, x = synth.layer_inputs(wl, 0, C=C)
    logits = torch.empty((C, wl.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((C, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((C, wl.k), dtype=torch.float32, device="cuda")
    rf().moe_route(to_dev(x), to_dev(Wr), logits, C, wl.H, wl.E, wl.k, idx, w,
                   _ws(wl.E, wl.H, 32, wl.k, C))
    L = oracle.router_logits(x, Wr)
    bound = oracle.logit_error_bound(x, Wr, route_depth(wl.H, C))
    Lg = logits.cpu().numpy().astype(np.float64)
    err = np.abs(Lg - L)
    say(f"  largest |fp32 - exact| / bound: {float(np.max(err / bound)):.3f}; "
        f"median bound {float(np.median(bound)):.2e}")
    assert np.all(err <= bound), "fp32 logits outside the certified bound"
    near = check_selection(L, idx.cpu().numpy(), bound, wl.k, steered=wl.routing == "zipf")
    say(f"  near-tie tokens: {near} of {C}")
    g = idx.cpu().numpy()
    wref = np.stack([oracle.route_weights(L[t, g[t]]) for t in range(C)])
    np.testing.assert_allclose(w.cpu().numpy(), wref, rtol=1e-3)


# ---------------------------------------------------------------------------
# Whole layer
# ---------------------------------------------------------------------------
def _layer(name, C=None, fmt=None, layer=0, pool=0):
    wl = synth.WORKLOADS[name]
    if fmt is not None:
        wl = wl.with_(fmt=fmt)
    C = wl.C if C is None else C
    spec = wl.bank(layer)
    bank = cached_bank(spec)
    Wr, x = synth.layer_inputs(wl, layer, pool=pool, C=C)
    out = torch.empty((C, wl.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((C, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((C, wl.k), dtype=torch.float32, device="cuda")
    ws = _ws(wl.E, wl.H, wl.I, wl.k, C)
    rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), C, wl.k, out, idx, w, ws)
    torch.cuda.synchronize()
    return wl, spec, bank, Wr, x, out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), ws


@pytest.mark.parametrize("name,C,fmt", [
    ("tiny", 4, None), ("tiny", 4, synth.FMT_NV), ("tiny", 1, None), ("tiny", 16, None),
    ("w50_k16", 1, None), ("w50_k8", 1, None), ("w50_c7_k8", 7, None), ("w50_c7_k16", 7, None),
    ("k3_stack", 1, None), ("k3_stack_zipf", 1, None),
])
def test_layer_parity(name, C, fmt):
    say(f"[layer] {name} C={C} fmt={fmt}")
    wl, spec, bank, Wr, x, out, idx, w, _ = _layer(name, C, fmt)
    L = oracle.router_logits(x, Wr)
    bound = oracle.logit_error_bound(x, Wr, route_depth(wl.H, C))
    near = check_selection(L, idx, bound, wl.k, steered=wl.routing == "zipf")
    say(f"  near-tie tokens: {near}; distinct experts: {len(np.unique(idx))}")
    ref = oracle.layer(spec, Wr, x, wl.k, idx=idx)
    assert_close(out, ref["out"], f"{name} C={C}")


def test_layer_k_equals_E_and_k1():
    say("[layer] tiny k=E and k=1")
    for k in (8, 1):
        wl = synth.WORKLOADS["tiny"].with_(k=k)
        spec = wl.bank(0)
        bank = cached_bank(spec)
        Wr, x = synth.layer_inputs(wl, 0)
        out = torch.empty((wl.C, wl.H), dtype=torch.float32, device="cuda")
        idx = torch.empty((wl.C, k), dtype=torch.int32, device="cuda")
        w = torch.empty((wl.C, k), dtype=torch.float32, device="cuda")
        rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), wl.C, k, out, idx, w,
                           _ws(wl.E, wl.H, wl.I, k, wl.C))
        ref = oracle.layer(spec, Wr, x, k)
        assert np.array_equal(idx.cpu().numpy(), ref["idx"])
        if k == 1:
            assert np.all(w.cpu().numpy() == 1.0)
        assert_close(out.cpu().numpy(), ref["out"], f"tiny k={k}")


def test_expert_fwd_given_selection_and_invalid_slots():
    """moe_expert_fwd with caller weights; slots naming experts outside [0, E)
    contribute nothing."""
    say("[expert_fwd] caller selection with invalid slots")
    wl = synth.WORKLOADS["tiny"]
    spec = wl.bank(0)
    bank = cached_bank(spec)
    _, x = synth.layer_inputs(wl, 0)
    idx = np.array([[1, 5], [5, -1], [8, 2], [-3, 100]], np.int32)
    w = np.array([[0.25, 0.75], [1.0, 0.5], [0.5, 0.5], [1.0, 1.0]], np.float32)
    out = torch.empty((wl.C, wl.H), dtype=torch.float32, device="cuda")
    rf().moe_expert_fwd(bank, to_dev(x), wl.C, wl.k, to_dev(idx), to_dev(w), out,
                        _ws(wl.E, wl.H, wl.I, wl.k, wl.C))
    valid = (idx >= 0) & (idx < wl.E)
    ref = oracle.experts_forward(spec, x, np.where(valid, idx, 0), np.where(valid, w, 0.0))
    got = out.cpu().numpy()
    assert np.all(got[3] == 0.0)
    assert_close(got[:3], ref[:3], "expert_fwd")


def test_layer_deterministic_and_down_scale_doubling():
    """Two runs are bit-identical; doubling every down-matrix e8m0 scale doubles
    the output bit-exactly (a power-of-two scaling commutes with rounding)."""
    say("[layer] determinism + down-scale doubling")
    wl = synth.WORKLOADS["tiny"]
    spec = wl.bank(0)
    bank = make_bank(spec)
    Wr, x = synth.layer_inputs(wl, 0)
    ws = _ws(wl.E, wl.H, wl.I, wl.k, wl.C)
    outs = []
    for _ in range(2):
        out = torch.empty((wl.C, wl.H), dtype=torch.float32, device="cuda")
        rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), wl.C, wl.k, out, ws=ws)
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    n = spec.tensor_bytes(5)
    for e in range(wl.E):
        v = bank.tensor_view(e, 5, n)
        v.add_(1)
    out = torch.empty((wl.C, wl.H), dtype=torch.float32, device="cuda")
    rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), wl.C, wl.k, out, ws=ws)
    assert np.array_equal(out.cpu().numpy(), 2 * outs[0])


def test_layer_identical_experts():
    """All experts share expert 3's bytes: the output no longer depends on the
    routing (the weights sum to one)."""
    say("[layer] identical experts")
    wl = synth.WORKLOADS["tiny"]
    spec = wl.bank(0)
    bank = make_bank(spec)
    rec = bank.storage[3 * bank.stride:(4) * bank.stride].clone()
    for e in range(wl.E):
        bank.storage[e * bank.stride:(e + 1) * bank.stride].copy_(rec)
    Wr, x = synth.layer_inputs(wl, 0)
    out = torch.empty((wl.C, wl.H), dtype=torch.float32, device="cuda")
    rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), wl.C, wl.k, out,
                       ws=_ws(wl.E, wl.H, wl.I, wl.k, wl.C))
    W = oracle.expert_weights(spec, 3)
    ref = np.stack([oracle.expert_ffn(*W, x[t]) for t in range(wl.C)])
    assert_close(out.cpu().numpy(), ref, "identical experts")


def test_workspace_reuse_across_shapes():
    """One workspace sized for the larger call serves a smaller one afterwards;
    the counters left behind by the first call are zero again."""
    say("[layer] workspace reuse")
    wl = synth.WORKLOADS["tiny"]
    spec = wl.bank(0)
    bank = cached_bank(spec)
    ws = _ws(wl.E, wl.H, wl.I, wl.k, 16)
    for C in (16, 3, 1):
        Wr, x = synth.layer_inputs(wl, 0, C=C, pool=C)
        out = torch.empty((C, wl.H), dtype=torch.float32, device="cuda")
        idx = torch.empty((C, wl.k), dtype=torch.int32, device="cuda")
        rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), C, wl.k, out, idx, None, ws)
        ref = oracle.layer(spec, Wr, x, wl.k)
        assert np.array_equal(idx.cpu().numpy(), ref["idx"])
        assert_close(out.cpu().numpy(), ref["out"], f"reuse C={C}")


@pytest.mark.parametrize("name,C", [("w50_k16", 1), ("w50_c7_k16", 7), ("k3_stack", 1)])
def test_layer_repeat_bit_identical(name, C):
    """60 back-to-back calls on one stream give bit-identical outputs: the
    cross-workgroup hand-offs (router partial sums, per-slot down outputs)
    are complete before the last workgroup sums them."""
    say(f"[layer] repeat x60 {name} C={C}")
    wl = synth.WORKLOADS[name]
    spec = wl.bank(0)
    bank = cached_bank(spec)
    Wr, x = synth.layer_inputs(wl, 0, C=C, pool=3)
    ws = _ws(wl.E, wl.H, wl.I, wl.k, C)
    Wr_d, x_d = to_dev(Wr), to_dev(x)
    outs = torch.empty((60, C, wl.H), dtype=torch.float32, device="cuda")
    idxs = torch.empty((60, C, wl.k), dtype=torch.int32, device="cuda")
    for i in range(60):
        rf().moe_layer_fwd(bank, Wr_d, x_d, C, wl.k, outs[i], idxs[i], None, ws)
    torch.cuda.synchronize()
    o = outs.cpu().numpy().view(np.uint32)
    ix = idxs.cpu().numpy()
    assert all(np.array_equal(o[0], o[i]) for i in range(60))
    assert all(np.array_equal(ix[0], ix[i]) for i in range(60))
    # no bounded wait of the decode kernel expired (the word at byte 16)
    assert int(ws.tensor[4].item()) == 0


# ---------------------------------------------------------------------------
# Batched path: C >= 2 tokens as grouped GEMMs on the matrix cores, and the
# matrix-core router for C > 16
# ---------------------------------------------------------------------------
def _small_prefill(C, fmt, routing):
    return synth.Workload(f"bsmall_{C}", fmt, 64, 8, 1024, 512, C, 1, routing,
                          1.0 if routing == "zipf" else 0.0, routing == "zipf")


@pytest.mark.parametrize("C,fmt,routing", [(2, synth.FMT_NV, "natural"), (17, synth.FMT_NV, "natural"),
                                           (65, synth.FMT_MX, "zipf"), (200, synth.FMT_NV, "zipf"),
                                           (200, synth.FMT_MX, "natural")])
def test_batched_layer_parity(C, fmt, routing):
    """64 experts, top-8, H 1024, I 512: tiles of 16 (C <= 64) or 64 tokens,
    hot experts spanning several tiles, partial last tiles; Zipf cases use
    bf16-exact activations (one activation plane), natural ones fp32 (three)."""
    wl = _small_prefill(C, fmt, routing)
    say(f"[batched] C={C} fmt={fmt} {routing}")
    _batched_layer_check(wl, routing)


@pytest.mark.parametrize("I,C,fmt,routing", [(1024, 200, synth.FMT_NV, "zipf"),
                                             (1536, 130, synth.FMT_MX, "natural"),
                                             (1536, 257, synth.FMT_NV, "zipf")])
def test_batched_persistent_down_parity(I, C, fmt, routing):
    """An inner width of four 256-wide K stages or more, where the down GEMM
    runs as persistent workgroups taking (tile, row block) items from a
    counter and loading each next item's first stages during the current
    one's last: 64 experts, top-8, H 1024 (two 512-row blocks), element by
    element.  Zipf cases put 181 and 235 tokens on the hottest expert (3 and
    4 tiles of 64, the last partial); natural routing gives many one-tile
    experts, so consecutive items change expert at almost every step."""
    wl = synth.Workload(f"bdnp_{I}_{C}", fmt, 64, 8, 1024, I, C, 1, routing,
                        1.0 if routing == "zipf" else 0.0, routing == "zipf")
    say(f"[batched, persistent down] I={I} C={C} fmt={fmt} {routing}")
    _batched_layer_check(wl, routing)


def _batched_layer_check(wl, routing):
    C = wl.C
    spec = wl.bank(0)
    bank = cached_bank(spec)
    Wr, x = synth.layer_inputs(wl, 0)
    out = torch.empty((C, wl.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((C, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((C, wl.k), dtype=torch.float32, device="cuda")
    rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), C, wl.k, out, idx, w,
                       _ws(wl.E, wl.H, wl.I, wl.k, C))
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    L = oracle.router_logits(x, Wr)
    near = check_selection(L, g, oracle.logit_error_bound(x, Wr, route_depth(wl.H, C)), wl.k,
                           steered=routing == "zipf")
    counts = np.bincount(g.ravel(), minlength=wl.E)
    say(f"  near-tie tokens: {near}; most tokens on one expert: {counts.max()}")
    wref = np.stack([oracle.route_weights(L[t, g[t]]) for t in range(C)])
    np.testing.assert_allclose(w.cpu().numpy(), wref, rtol=1e-5)
    ref = oracle.layer(spec, Wr, x, wl.k, idx=g)
    assert_close(out.cpu().numpy(), ref["out"], f"batched C={C}")


def test_batched_repeat_bit_identical():
    """The grouping of pairs into tiles depends on atomics, but each output is
    a fixed-order sum over its own row: repeated calls are bit-identical."""
    wl = _small_prefill(200, synth.FMT_NV, "zipf")
    say("[batched] repeat x10 C=200")
    bank = cached_bank(wl.bank(0))
    Wr, x = synth.layer_inputs(wl, 0)
    ws = _ws(wl.E, wl.H, wl.I, wl.k, wl.C)
    Wr_d, x_d = to_dev(Wr), to_dev(x)
    outs = torch.empty((10, wl.C, wl.H), dtype=torch.float32, device="cuda")
    for i in range(10):
        rf().moe_layer_fwd(bank, Wr_d, x_d, wl.C, wl.k, outs[i], None, None, ws)
    torch.cuda.synchronize()
    o = outs.cpu().numpy().view(np.uint32)
    assert all(np.array_equal(o[0], o[i]) for i in range(10))


def test_prefill_k3_full_size_sampled():
    """The K3 prefill shape at full size: 896 experts, top-16, H 7168, I 1536,
    NVFP4, 2048 bf16-exact tokens with Zipf s=1.0 routing.  The whole selection
    is checked against the oracle's fp64 router; the outputs of sampled tokens
    (among them tokens of the most loaded expert) against the oracle."""
    wl = synth.WORKLOADS["k3_prefill"]
    say(f"[prefill] K3 full size T={wl.C}")
    spec = wl.bank(0)
    bank = make_bank(spec)
    Wr, x = synth.layer_inputs(wl, 0)
    C = wl.C
    out = torch.empty((C, wl.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((C, wl.k), dtype=torch.int32, device="cuda")
    w = torch.empty((C, wl.k), dtype=torch.float32, device="cuda")
    rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), C, wl.k, out, idx, w,
                       _ws(wl.E, wl.H, wl.I, wl.k, C))
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    say("  oracle router over all tokens")
    L = oracle.router_logits(x, Wr)
    near = check_selection(L, g, oracle.logit_error_bound(x, Wr, route_depth(wl.H, C)), wl.k,
                           steered=True)
    counts = np.bincount(g.ravel(), minlength=wl.E)
    hot = int(np.argmax(counts))
    say(f"  near-tie tokens: {near}; experts touched {np.count_nonzero(counts)}; "
        f"hottest expert {hot} with {counts.max()} tokens")
    hot_tokens = np.nonzero((g == hot).any(axis=1))[0]
    sample = sorted({0, C - 1, int(hot_tokens[0]), int(hot_tokens[-1])})
    got = out.cpu().numpy()
    for t in sample:                    # one token at a time: 16 experts in host memory
        ref = oracle.layer(spec, Wr, x[[t]], wl.k, idx=g[[t]])
        assert_close(got[[t]], ref["out"], f"prefill token {t}")


def test_layer_k3_natural_c64_sampled():
    """The K3 shape (896 experts, top-16, H 7168, I 1536, NVFP4) at 64 tokens
    of natural (unsteered) routing: the matrix-core router and top-k for all
    tokens against the oracle within the certified bound, and sampled tokens'
    outputs (among them one of the most loaded expert) against the oracle."""
    wl = synth.WORKLOADS["k3_stack"]
    C = 64
    say(f"[batched] K3 shape, natural routing, C={C}")
    spec = wl.bank(0)
    bank = cached_bank(spec)
    Wr, x = synth.layer_inputs(wl, 0, C=C, pool=1)
    out = torch.empty((C, wl.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((C, wl.k), dtype=torch.int32, device="cuda")
    rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), C, wl.k, out, idx, None,
                       _ws(wl.E, wl.H, wl.I, wl.k, C))
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    L = oracle.router_logits(x, Wr)
    near = check_selection(L, g, oracle.logit_error_bound(x, Wr, route_depth(wl.H, C)), wl.k)
    counts = np.bincount(g.ravel(), minlength=wl.E)
    hot = int(np.argmax(counts))
    say(f"  near-tie tokens: {near}; distinct experts {np.count_nonzero(counts)}; "
        f"hottest expert {hot} with {counts.max()} tokens")
    hot_tokens = np.nonzero((g == hot).any(axis=1))[0]
    got = out.cpu().numpy()
    cache = {}
    for t in sorted({0, int(hot_tokens[0]), C - 1}):
        ref = oracle.experts_forward(spec, x[[t]], g[[t]],
                                     np.stack([oracle.route_weights(L[t, g[t]])]), cache)
        assert_close(got[[t]], ref, f"K3 natural C=64 token {t}")


def test_batched_expert_fwd_invalid_and_repeated_slots():
    """The batched path with a caller selection: slots naming experts outside
    [0, E) contribute nothing, an expert named twice by one token counts
    twice, and a token whose slots are all invalid gets zeros."""
    wl = _small_prefill(5, synth.FMT_NV, "natural")
    say("[batched] expert_fwd with invalid and repeated slots, C=5")
    spec = wl.bank(0)
    bank = cached_bank(spec)
    _, x = synth.layer_inputs(wl, 0)
    rng = np.random.default_rng(11)
    idx = rng.integers(0, wl.E, size=(wl.C, wl.k)).astype(np.int32)
    idx[0, 3] = -1
    idx[1, :2] = 17                      # the same expert in two slots
    idx[2, 5] = wl.E
    idx[4, :] = -7                       # no valid slot at all
    w = rng.uniform(0.05, 1.0, size=(wl.C, wl.k)).astype(np.float32)
    out = torch.empty((wl.C, wl.H), dtype=torch.float32, device="cuda")
    rf().moe_expert_fwd(bank, to_dev(x), wl.C, wl.k, to_dev(idx), to_dev(w), out,
                        _ws(wl.E, wl.H, wl.I, wl.k, wl.C))
    valid = (idx >= 0) & (idx < wl.E)
    ref = oracle.experts_forward(spec, x, np.where(valid, idx, 0), np.where(valid, w, 0.0))
    got = out.cpu().numpy()
    assert np.all(got[4] == 0.0)
    assert_close(got[:4], ref[:4], "batched expert_fwd")


@pytest.mark.parametrize("ties", [448, 70])
def test_decode_kernel_clustered_winners(ties):
    """The one-launch decode kernel (W50 shape, top-16) when more than 64
    experts share the threshold: the first `ties` router rows are identical,
    so their logits tie exactly above all others (the rest are scaled down),
    and the top 16 are the tied experts of lowest index.  Selection
    bit-exact with the oracle, output within the bar."""
    wl = synth.WORKLOADS["w50_k16"]
    say(f"[decode] clustered winners: {ties} tied logits")
    spec = wl.bank(0)
    bank = cached_bank(spec)
    Wr, x = synth.layer_inputs(wl, 0, C=1)
    Wr = Wr.copy()
    row = np.abs(Wr[0]) * np.sign(x[0])          # a row with a large positive logit
    Wr[:ties] = row
    Wr[ties:] *= 0.01
    out = torch.empty((1, wl.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((1, wl.k), dtype=torch.int32, device="cuda")
    rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), 1, wl.k, out, idx, None,
                       _ws(wl.E, wl.H, wl.I, wl.k, 1))
    torch.cuda.synchronize()
    ref = oracle.layer(spec, Wr, x, wl.k)
    assert ref["idx"][0].tolist() == list(range(wl.k))
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    assert_close(out.cpu().numpy(), ref["out"], f"clustered winners ({ties} ties)")


def test_decode_expert_fwd_invalid_and_repeated_slots():
    """The one-launch decode kernel with a caller selection (W50 shape, top-16):
    an invalid slot contributes nothing and a repeated expert counts twice."""
    wl = synth.WORKLOADS["w50_k16"]
    say("[decode] expert_fwd with invalid and repeated slots, W50 top-16")
    spec = wl.bank(0)
    bank = cached_bank(spec)
    _, x = synth.layer_inputs(wl, 0, C=1)
    rng = np.random.default_rng(12)
    idx = rng.choice(wl.E, size=(1, wl.k), replace=False).astype(np.int32)
    idx[0, 4] = -1
    idx[0, 9] = idx[0, 2]
    idx[0, 15] = wl.E + 3
    w = rng.uniform(0.01, 0.2, size=(1, wl.k)).astype(np.float32)
    out = torch.empty((1, wl.H), dtype=torch.float32, device="cuda")
    rf().moe_expert_fwd(bank, to_dev(x), 1, wl.k, to_dev(idx), to_dev(w), out,
                        _ws(wl.E, wl.H, wl.I, wl.k, 1))
    valid = (idx >= 0) & (idx < wl.E)
    ref = oracle.experts_forward(spec, x, np.where(valid, idx, 0), np.where(valid, w, 0.0))
    assert_close(out.cpu().numpy(), ref, "decode expert_fwd")


@pytest.mark.parametrize("E,k,C", [(64, 1, 33), (32, 32, 3)])
def test_batched_k1_and_k_equals_E(E, k, C):
    """Batched path at the degenerate top-k values: k = 1 (every weight is 1)
    and k = E = 32 (every token uses every expert)."""
    wl = _small_prefill(C, synth.FMT_MX, "natural").with_(E=E, k=k)
    say(f"[batched] k={k} C={C}")
    spec = wl.bank(0)
    bank = cached_bank(spec)
    Wr, x = synth.layer_inputs(wl, 0)
    out = torch.empty((C, wl.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((C, k), dtype=torch.int32, device="cuda")
    w = torch.empty((C, k), dtype=torch.float32, device="cuda")
    rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), C, k, out, idx, w, _ws(wl.E, wl.H, wl.I, k, C))
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    L = oracle.router_logits(x, Wr)
    check_selection(L, g, oracle.logit_error_bound(x, Wr, route_depth(wl.H, C)), k)
    if k == 1:
        assert np.all(w.cpu().numpy() == 1.0)
    else:
        assert all(sorted(row) == list(range(wl.E)) for row in g.tolist())
    ref = oracle.layer(spec, Wr, x, k, idx=g)
    assert_close(out.cpu().numpy(), ref["out"], f"batched k={k}")


def test_batched_max_tokens_sampled():
    """The largest call the library takes (MOE_MAX_TOKENS tokens) on the small
    batched shape with Zipf routing: the whole selection is checked against
    the oracle's router, sampled tokens' outputs against the oracle."""
    C = rf().MOE_MAX_TOKENS
    wl = _small_prefill(C, synth.FMT_NV, "zipf")
    say(f"[batched] C={C} (maximum)")
    spec = wl.bank(0)
    bank = cached_bank(spec)
    Wr, x = synth.layer_inputs(wl, 0)
    out = torch.empty((C, wl.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((C, wl.k), dtype=torch.int32, device="cuda")
    rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), C, wl.k, out, idx, None,
                       _ws(wl.E, wl.H, wl.I, wl.k, C))
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    L = oracle.router_logits(x, Wr)
    check_selection(L, g, oracle.logit_error_bound(x, Wr, route_depth(wl.H, C)), wl.k, steered=True)
    counts = np.bincount(g.ravel(), minlength=wl.E)
    hot = int(np.argmax(counts))
    hot_tokens = np.nonzero((g == hot).any(axis=1))[0]
    say(f"  hottest expert {hot} with {counts.max()} tokens")
    got = out.cpu().numpy()
    for t in sorted({0, 1, C // 2, C - 1, int(hot_tokens[0]), int(hot_tokens[-1])}):
        ref = oracle.layer(spec, Wr, x[[t]], wl.k, idx=g[[t]])
        assert_close(got[[t]], ref["out"], f"max-tokens token {t}")


# ---------------------------------------------------------------------------
# Decode batches (C = 2..16): each distinct expert streamed once
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("C,k,fmt", [(16, 8, synth.FMT_NV), (16, 32, synth.FMT_MX), (9, 4, synth.FMT_MX),
                                     (1, 8, synth.FMT_NV), (2, 1, synth.FMT_MX)])
def test_decode_batch_passes_and_limits(C, k, fmt):
    """64 experts, H 1024, I 512, fp32 tokens with Zipf routing: experts chosen
    by more tokens than one activation pass holds (8) take several passes over
    their weights; C = 16 with k = 32 is the largest pair count (512); C = 1
    (a shape the one-launch kernel is not built for) selects in the router's
    last workgroup; k = 1."""
    wl = synth.Workload(f"dsmall_{C}_{k}", fmt, 64, k, 1024, 512, C, 1, "zipf", 1.0, False)
    say(f"[decode batch] C={C} k={k} fmt={fmt}")
    spec = wl.bank(0)
    bank = cached_bank(spec)
    Wr, x = synth.layer_inputs(wl, 0)
    out = torch.empty((C, wl.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((C, k), dtype=torch.int32, device="cuda")
    w = torch.empty((C, k), dtype=torch.float32, device="cuda")
    rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), C, k, out, idx, w, _ws(wl.E, wl.H, wl.I, k, C))
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    L = oracle.router_logits(x, Wr)
    check_selection(L, g, oracle.logit_error_bound(x, Wr, route_depth(wl.H, C)), k, steered=True)
    counts = np.bincount(g.ravel(), minlength=wl.E)
    say(f"  most tokens on one expert: {counts.max()}; distinct experts: {np.count_nonzero(counts)}")
    if C == 16:
        assert counts.max() > 8                   # the multi-pass case is exercised
    wref = np.stack([oracle.route_weights(L[t, g[t]]) for t in range(C)])
    np.testing.assert_allclose(w.cpu().numpy(), wref, rtol=1e-5)
    ref = oracle.layer(spec, Wr, x, k, idx=g)
    assert_close(out.cpu().numpy(), ref["out"], f"decode batch C={C} k={k}")


def test_decode_batch_k3_shape_sampled():
    """The K3 shape (H 7168: four pairs per gate/up activation pass) with 12
    tokens and Zipf 1.2 routing; sampled tokens, among them two of the most
    loaded expert, against the oracle."""
    wl = synth.WORKLOADS["k3_stack_zipf"]
    C = 12
    say(f"[decode batch] K3 shape C={C}")
    spec = wl.bank(0)
    bank = cached_bank(spec)
    Wr, x = synth.layer_inputs(wl, 0, C=C)
    out = torch.empty((C, wl.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((C, wl.k), dtype=torch.int32, device="cuda")
    rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), C, wl.k, out, idx, None,
                       _ws(wl.E, wl.H, wl.I, wl.k, C))
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    L = oracle.router_logits(x, Wr)
    check_selection(L, g, oracle.logit_error_bound(x, Wr, route_depth(wl.H, C)), wl.k, steered=True)
    counts = np.bincount(g.ravel(), minlength=wl.E)
    hot = int(np.argmax(counts))
    say(f"  hottest expert {hot} with {counts.max()} tokens")
    assert counts.max() > 4                       # more than one gate/up pass
    hot_tokens = np.nonzero((g == hot).any(axis=1))[0]
    got = out.cpu().numpy()
    for t in sorted({0, int(hot_tokens[0]), int(hot_tokens[-1])}):
        ref = oracle.layer(spec, Wr, x[[t]], wl.k, idx=g[[t]])
        assert_close(got[[t]], ref["out"], f"K3 decode batch token {t}")


@pytest.mark.parametrize("E,k,H,I,C,fmt", [(16, 4, 512, 512, 6, synth.FMT_NV), (1024, 32, 512, 1024, 16, synth.FMT_MX)])
def test_decode_batch_shape_limits(E, k, H, I, C, fmt):
    """The smallest rows the decode-batch streams take (one 256-byte chunk per
    row at H = 512) and the largest distinct-expert count (1024 experts,
    top-32, 16 tokens: up to 512 distinct experts)."""
    wl = synth.Workload(f"dlim_{E}_{k}_{H}", fmt, E, k, H, I, C, 1, "natural", 0.0, False)
    say(f"[decode batch] E={E} k={k} H={H} I={I} C={C}")
    spec = wl.bank(0)
    bank = cached_bank(spec)
    Wr, x = synth.layer_inputs(wl, 0)
    out = torch.empty((C, H), dtype=torch.float32, device="cuda")
    idx = torch.empty((C, k), dtype=torch.int32, device="cuda")
    rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), C, k, out, idx, None, _ws(E, H, I, k, C))
    torch.cuda.synchronize()
    g = idx.cpu().numpy()
    L = oracle.router_logits(x, Wr)
    check_selection(L, g, oracle.logit_error_bound(x, Wr, route_depth(H, C)), k)
    say(f"  distinct experts: {len(np.unique(g))}")
    ref = oracle.layer(spec, Wr, x, k, idx=g)
    assert_close(out.cpu().numpy(), ref["out"], f"decode batch E={E} k={k} H={H}")
