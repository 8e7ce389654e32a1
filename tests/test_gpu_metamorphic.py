"""Metamorphic checks of the HIP path that need no oracle value: properties
the method fixes whatever the data.

* MX bank re-encoded as NV: every e8m0 block scale 2^(b-127) becomes two
  e4m3 block scales of the same value (exact for the bank's bytes) and the
  per-tensor scales are 1.  moe_dequant must give bit-identical matrices, the
  selection must not change, and the layer outputs of the two banks must
  agree within the parity bar (the two formats take different kernel
  instances).
* Experts relabelled together with their router rows: the fp32 logits are
  permuted, so the selection is the permuted one and the output is
  bit-identical (the expert work and the combine do not depend on the ids).

Both run through the C ABI on the decode kernel (one token), the decode-batch
streams (2..16 tokens) and the matrix-core tiles (more tokens).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, make_bank, say, to_dev

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


def _tensor(bank, t, shape):
    """[E][...] view of tensor t of every expert."""
    n = int(np.prod(shape))
    rec = bank.storage.view(bank.E, bank.stride)
    return rec[:, bank.offsets[t]:bank.offsets[t] + n].view(bank.E, *shape)


def _mx_as_nv(mx):
    """The NV bank holding the same weights as the MX bank."""
    R = rf()
    nv = R.Bank(synth.FMT_NV, mx.E, mx.H, mx.I)
    nv.storage.zero_()
    H, I = mx.H, mx.I
    code_shapes = {0: (I, H // 2), 1: (I, H // 2), 2: (H, I // 2)}
    for t, shp in code_shapes.items():
        _tensor(nv, t, shp).copy_(_tensor(mx, t, shp))
    for t, (N, K) in {3: (I, H), 4: (I, H), 5: (H, I)}.items():
        b = _tensor(mx, t, (N, K // 32)).to(torch.int32)
        assert int(b.min()) >= 121 and int(b.max()) <= 135      # e4m3 normal range 2^-6 .. 2^8
        e4m3 = ((b - 120) * 8).to(torch.uint8)                   # 2^(b-127): exponent field b-120, mantissa 0
        _tensor(nv, t, (N, K // 16)).copy_(e4m3.repeat_interleave(2, dim=2))
    ones = torch.ones((mx.E, 3), dtype=torch.float32, device="cuda").view(torch.uint8)
    _tensor(nv, 6, (12,)).copy_(ones)
    torch.cuda.synchronize()
    return nv


def _layer(bank, Wr, x, k):
    C, H = x.shape
    out = torch.empty((C, H), dtype=torch.float32, device="cuda")
    idx = torch.empty((C, k), dtype=torch.int32, device="cuda")
    ws = rf().Workspace(bank.E, H, bank.I, k, C)
    rf().moe_layer_fwd(bank, to_dev(Wr), to_dev(x), C, k, out, idx, None, ws)
    torch.cuda.synchronize()
    assert int(ws.tensor[4].item()) == 0          # no bounded wait expired
    return out.cpu().numpy(), idx.cpu().numpy()


# (name, workload, token counts): the W50 shape takes the decode kernel at one
# token; the small shape the decode-batch streams and the matrix-core tiles
MX_CASES = [("w50_k16", synth.WORKLOADS["w50_k16"], (1,)),
            ("small", synth.Workload("meta_small", synth.FMT_MX, 64, 8, 1024, 512, 40, 1, "natural",
                                     0.0, False), (5, 40, 100))]


@pytest.mark.parametrize("name,wl,Cs", MX_CASES)
def test_mx_bank_reencoded_as_nv(name, wl, Cs):
    say(f"[metamorphic] MX bank as NV: {name}")
    mx = make_bank(wl.bank(0))
    nv = _mx_as_nv(mx)
    for e in (0, wl.E // 2, wl.E - 1):
        for m in range(3):
            N, K = (wl.H, wl.I) if m == 2 else (wl.I, wl.H)
            a = torch.empty((N, K), dtype=torch.float32, device="cuda")
            b = torch.empty((N, K), dtype=torch.float32, device="cuda")
            rf().moe_dequant(mx, e, m, a)
            rf().moe_dequant(nv, e, m, b)
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (e, m)
    for C in Cs:
        Wr, x = synth.layer_inputs(wl, 0, C=C)
        o_mx, i_mx = _layer(mx, Wr, x, wl.k)
        o_nv, i_nv = _layer(nv, Wr, x, wl.k)
        assert np.array_equal(i_mx, i_nv), f"C={C}: the selection depends on the bank"
        assert_close(o_nv, o_mx.astype(np.float64), f"{name} C={C}: NV bank against MX bank")
    del mx, nv
    torch.cuda.empty_cache()


REL_CASES = [("k3_stack", synth.WORKLOADS["k3_stack"], (1,)),
             ("w50_c7_k8", synth.WORKLOADS["w50_c7_k8"], (7,)),
             ("small_nv", synth.Workload("meta_small_nv", synth.FMT_NV, 64, 8, 1024, 512, 40, 1,
                                         "natural", 0.0, False), (3, 40, 100))]


@pytest.mark.parametrize("name,wl,Cs", REL_CASES)
def test_relabelled_experts_bit_identical(name, wl, Cs):
    say(f"[metamorphic] experts relabelled with their router rows: {name}")
    R = rf()
    bank = make_bank(wl.bank(0))
    perm = np.random.default_rng(5).permutation(wl.E)          # expert e -> perm[e]
    moved = R.Bank(wl.fmt, wl.E, wl.H, wl.I)
    src = bank.storage.view(wl.E, bank.stride)
    dst = moved.storage.view(wl.E, moved.stride)
    dst[torch.from_numpy(perm).to("cuda")] = src
    torch.cuda.synchronize()
    for C in Cs:
        Wr, x = synth.layer_inputs(wl, 0, C=C)
        Wr_p = np.empty_like(Wr)
        Wr_p[perm] = Wr
        o1, i1 = _layer(bank, Wr, x, wl.k)
        o2, i2 = _layer(moved, Wr_p, x, wl.k)
        assert np.array_equal(perm[i1], i2), f"C={C}: selection not the relabelled one"
        assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)), f"C={C}: output changed"
        say(f"  C={C}: bit-identical")
    del bank, moved
    torch.cuda.empty_cache()
