"""GPU parity of the MXFP4 path on the block-scaled FP4 matrix cores
(moe_expert_fwd_mx_mma) against the oracle, through the C ABI.

The instruction itself is not exact: it truncates the products of each group
of 8 below 2^(largest exponent sum - 13) (measured; modelled in
tests/fp4_mfma_model.py).  The activation terms are built so that no product
of a group falls below that quantum, so with 4 or more terms the path is held
to the library's bar: rel-L2 <= 2e-5 and max-abs <= 1e-4 * max|ref| of the
oracle's fp64 result.  Fewer terms are lossy by design: their measured error
is printed and bounded loosely."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import RTOL_L2, RTOL_MAX, cached_bank, say, to_dev


def assert_floor(got, ref, what):
    """The library's bar (near-exact mode, 4 or more terms)."""
    r, m = oracle.rel_l2(got, ref), oracle.max_abs_ratio(got, ref)
    say(f"  {what}: rel_l2 {r:.3e}  max_abs/max|ref| {m:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert r <= RTOL_L2 and m <= RTOL_MAX, f"{what}: rel_l2 {r:.3e} max {m:.3e}"

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


def _run(wl, terms, idx=None, x=None, Wr=None):
    """GPU output, x, oracle selection (idx, w)."""
    R = rf()
    spec = wl.bank(0)
    bank = cached_bank(spec)
    if x is None:
        Wr, x = synth.layer_inputs(wl, 0)
    C = x.shape[0]
    if idx is None:
        _, idx, w = oracle.route(x, Wr, wl.k)
    else:
        L = oracle.router_logits(x, Wr)
        w = np.stack([oracle.route_weights(L[t, np.clip(idx[t], 0, wl.E - 1)]) for t in range(C)])
    out = torch.empty((C, wl.H), dtype=torch.float32, device="cuda")
    ws = R.MxMmaWorkspace(bank, wl.k, C, terms)
    R.moe_expert_fwd_mx_mma(bank, to_dev(x), C, wl.k, to_dev(np.asarray(idx, np.int32)),
                            to_dev(np.asarray(w, np.float32)), out, terms, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), x, np.asarray(idx, np.int32), w, spec


@pytest.mark.parametrize("C,terms,bf16", [(40, 5, False), (200, 4, True), (3, 4, False), (70, 6, True)])
def test_mx_mma_parity(C, terms, bf16):
    wl = synth.Workload(f"mxm_{C}", synth.FMT_MX, 16, 4, 512, 768, C, 1, "zipf", 1.0, bf16)
    say(f"[mx mma] E=16 k=4 H=512 I=768 C={C} terms={terms} bf16_x={bf16}")
    got, x, idx, w, spec = _run(wl, terms)
    counts = np.bincount(idx.ravel(), minlength=wl.E)
    say(f"  most pairs on one expert: {counts.max()}")
    ref = oracle.experts_forward(spec, x, idx, w)
    assert_floor(got, ref, f"mx mma C={C} terms={terms}")


def test_mx_mma_single_term_lossy():
    """One e4m3 term per activation: the error of rounding x and h to 4
    significant bits under a shared block scale, measured and bounded
    loosely; more terms shrink it."""
    wl = synth.Workload("mxm_lossy", synth.FMT_MX, 16, 4, 512, 768, 40, 1, "zipf", 1.0, False)
    errs = []
    for terms in (1, 2, 3, 4):
        got, x, idx, w, spec = _run(wl, terms)
        ref = oracle.experts_forward(spec, x, idx, w)
        errs.append(oracle.rel_l2(got, ref))
        say(f"  terms={terms}: rel_l2 {errs[-1]:.3e}  max_abs/max|ref| {oracle.max_abs_ratio(got, ref):.3e}")
    assert errs[0] < 0.1
    assert errs[1] < errs[0] / 8 and errs[2] < errs[1] / 8
    assert errs[3] <= RTOL_L2


def test_mx_mma_w50_shape_sampled():
    """The W50 expert shape (448 experts, H 3584, I 3072, MXFP4) with 96
    bf16-exact tokens at top-8 and Zipf 1.0 routing, four terms; three tokens
    against the oracle, among them one of the most loaded expert."""
    wl = synth.Workload("mxm_w50", synth.FMT_MX, 448, 8, 3584, 3072, 96, 1, "zipf", 1.0, True)
    say("[mx mma] W50 shape C=96 terms=4")
    got, x, idx, w, spec = _run(wl, 4)
    counts = np.bincount(idx.ravel(), minlength=wl.E)
    hot = int(np.argmax(counts))
    say(f"  hottest expert {hot} with {counts.max()} pairs")
    assert counts.max() > 16
    hot_tokens = np.nonzero((idx == hot).any(axis=1))[0]
    cache = {}
    for t in sorted({0, int(hot_tokens[0]), 95}):
        ref = oracle.experts_forward(spec, x[[t]], idx[[t]], w[[t]], cache)
        assert_floor(got[[t]], ref, f"W50 mx mma token {t}")


def test_mx_mma_invalid_slots_and_limits():
    """Out-of-range expert indices contribute zero; NVFP4 banks, terms 0 and 7
    and shapes off the 256-row grid are refused."""
    R = rf()
    wl = synth.Workload("mxm_inv", synth.FMT_MX, 16, 4, 512, 768, 24, 1, "zipf", 1.0, False)
    Wr, x = synth.layer_inputs(wl, 0)
    _, idx, _ = oracle.route(x, Wr, wl.k)
    bad = idx.copy()
    bad[3, 1] = -1
    bad[7, 0] = 16
    bad[11, 2] = 1 << 20
    got, _, _, w, spec = _run(wl, 5, idx=bad, x=x, Wr=Wr)
    keep = (bad >= 0) & (bad < wl.E)
    ref = np.stack([oracle.combine(w[t][keep[t]], np.stack(
        [oracle.expert_ffn(*oracle.expert_weights(spec, int(e)), x[t]) for e in bad[t][keep[t]]]))
        for t in range(x.shape[0])])
    assert_floor(got, ref, "mx mma with invalid slots")
    bank = cached_bank(wl.bank(0))
    assert R.lib().moe_mx_mma_workspace_size(R._bank(bank), 4, 24, 0) == 0
    assert R.lib().moe_mx_mma_workspace_size(R._bank(bank), 4, 24, 7) == 0
    nv = cached_bank(wl.with_(fmt=synth.FMT_NV).bank(0))
    assert R.lib().moe_mx_mma_workspace_size(R._bank(nv), 4, 24, 2) == 0
    odd = cached_bank(synth.BankSpec(synth.FMT_MX, 8, 384, 512, 0, 0))
    assert R.lib().moe_mx_mma_workspace_size(R._bank(odd), 4, 24, 2) == 0


def test_mx_mma_repeat_bit_identical():
    wl = synth.Workload("mxm_rep", synth.FMT_MX, 16, 4, 512, 768, 100, 1, "zipf", 1.0, True)
    a, *_ = _run(wl, 4)
    b, *_ = _run(wl, 4)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("terms", [4, 1])
def test_mx_mma_w50_prefill_full_size_sampled(terms):
    """The bench's FP4 matrix-core configuration at full size: one 2048-token
    bf16-exact chunk through the W50 MXFP4 layer (448 experts, top-8, Zipf
    1.0); token 0, the first and last tokens of the most loaded expert, and
    the last token against the oracle.  Four terms: the library's bar;
    one term: the lossy mode's bound."""
    wl = synth.WORKLOADS["w50_prefill"]
    say(f"[mx mma] W50 prefill chunk C={wl.C} terms={terms}")
    got, x, idx, w, spec = _run(wl, terms)
    counts = np.bincount(idx.ravel(), minlength=wl.E)
    hot = int(np.argmax(counts))
    say(f"  hottest expert {hot} with {counts.max()} pairs, {int((counts > 0).sum())} experts touched")
    assert counts.max() > 64                      # several 64-pair tiles for one expert
    hot_tokens = np.nonzero((idx == hot).any(axis=1))[0]
    cache = {}
    for t in sorted({0, int(hot_tokens[0]), int(hot_tokens[-1]), wl.C - 1}):
        ref = oracle.experts_forward(spec, x[[t]], idx[[t]], w[[t]], cache)
        if terms >= 4:
            assert_floor(got[[t]], ref, f"W50 prefill token {t}")
        else:
            r = oracle.rel_l2(got[[t]], ref)
            say(f"  W50 prefill token {t} (1 term): rel_l2 {r:.3e}")
            assert r < 0.1
