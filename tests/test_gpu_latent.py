"""GPU parity of the latent MoE layer (router on x, routed_down, routed
experts in the latent space, RMS norm of their sum, routed_up, shared experts)
against the oracle, through the C ABI.  Same bars as the expert layer:
routing bit-exact up to certified near-ties, fp32 outputs within rel-L2 2e-5
and max-abs 1e-4 of the largest output.  Each case also checks the shared
part alone (gamma = 0) and that the routed part is not negligible beside it,
so the output bar covers both."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import assert_close, cached_bank, check_selection, route_depth, say, to_dev

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


def _bits(a):
    return to_dev(np.ascontiguousarray(a).view(np.int16))


def _run(wl, C, gamma_zero=False, ws=None):
    """(x, Wr, Wd, Wu, gamma, out, idx) of one GPU call."""
    R = rf()
    Wr, x, Wd, Wu, g = synth.latent_inputs(wl, 0, C=C)
    if gamma_zero:
        g = np.zeros_like(g)
    layer = R.LatentLayer(to_dev(Wr), _bits(Wd), to_dev(g), wl.eps, _bits(Wu),
                          cached_bank(wl.routed_bank()), cached_bank(wl.shared_bank()))
    ws = R.LatentWorkspace(layer, wl.k, C) if ws is None else ws
    out = torch.empty((C, wl.H), dtype=torch.float32, device="cuda")
    idx = torch.empty((C, wl.k), dtype=torch.int32, device="cuda")
    R.moe_latent_layer_fwd(layer, to_dev(x), C, wl.k, out, idx, None, ws)
    torch.cuda.synchronize()
    return x, Wr, Wd, Wu, g, out.cpu().numpy(), idx.cpu().numpy()


def _rms(a):
    return float(np.sqrt(np.mean(np.square(a))))


def _small(fmt, C, k=8, ns=2):
    return synth.LatentWorkload(f"lat_small_{C}", fmt, 64, k, 1024, 512, 512, ns, 1024, C,
                                gamma_scale=2.0 ** 17)


@pytest.mark.parametrize("C,fmt,k,ns", [(1, synth.FMT_NV, 8, 2), (1, synth.FMT_MX, 4, 3),
                                        (5, synth.FMT_MX, 8, 2), (16, synth.FMT_NV, 16, 3),
                                        (3, synth.FMT_MX, 1, 1)])
def test_latent_layer_parity(C, fmt, k, ns):
    wl = _small(fmt, C, k, ns)
    say(f"[latent] E={wl.E} k={k} H={wl.H} L={wl.L} shared={ns} C={C} fmt={fmt}")
    x, Wr, Wd, Wu, g, out, idx = _run(wl, C)
    L = oracle.router_logits(x, Wr)
    near = check_selection(L, idx, oracle.logit_error_bound(x, Wr, route_depth(wl.H, C)), k)
    say(f"  near-tie tokens: {near}")
    ref = oracle.latent_layer(wl, Wr, x, Wd, Wu, g, idx=idx)
    assert _rms(ref["routed"]) > 0.1 * _rms(ref["shared"])
    assert_close(out, ref["out"], f"latent C={C}")
    _, _, _, _, _, shared, _ = _run(wl, C, gamma_zero=True)
    assert_close(shared, ref["shared"], f"latent shared part C={C}")


def test_latent_workspace_reuse_and_limits():
    """One workspace sized for 16 tokens serves a 16-token call and then a
    2-token one; unsupported shapes are refused with MOE_ERR_UNSUPPORTED."""
    R = rf()
    wl = _small(synth.FMT_MX, 16)
    say("[latent] workspace reuse 16 -> 2 tokens")
    Wr, x, Wd, Wu, g = synth.latent_inputs(wl, 0, C=16)
    layer = R.LatentLayer(to_dev(Wr), _bits(Wd), to_dev(g), wl.eps, _bits(Wu),
                          cached_bank(wl.routed_bank()), cached_bank(wl.shared_bank()))
    ws = R.LatentWorkspace(layer, wl.k, 16)
    for C in (16, 2):
        out = torch.empty((C, wl.H), dtype=torch.float32, device="cuda")
        idx = torch.empty((C, wl.k), dtype=torch.int32, device="cuda")
        R.moe_latent_layer_fwd(layer, to_dev(x[:C]), C, wl.k, out, idx, None, ws)
        torch.cuda.synchronize()
        ref = oracle.latent_layer(wl, Wr, x[:C], Wd, Wu, g, idx=idx.cpu().numpy())
        assert_close(out.cpu().numpy(), ref["out"], f"latent reuse C={C}")
    out = torch.empty((17, wl.H), dtype=torch.float32, device="cuda")
    assert R.lib().moe_latent_workspace_size(R.ctypes.byref(layer.struct), wl.k, 17) == 0
    with pytest.raises(R.MoeError):
        R.moe_latent_layer_fwd(layer, to_dev(np.zeros((17, wl.H), np.float32)), 17, wl.k, out,
                               None, None, ws)


_K3_WEIGHTS = {"routed": {}, "shared": {}}     # dequantised experts, shared by both cases


@pytest.mark.parametrize("C", [1, 4])
def test_latent_k3_shape_token0(C):
    """The K3 latent shape (896 routed experts, top-16, H 7168, latent 3584,
    FFN 3072, 2 shared experts, NVFP4): one token through the single-launch
    expert kernel, and four tokens through the decode-batch streams; token 0
    against the oracle."""
    wl = synth.LATENT_WORKLOADS["k3_latent"]
    say(f"[latent] K3 shape C={C}")
    x, Wr, Wd, Wu, g, out, idx = _run(wl, C)
    L = oracle.router_logits(x, Wr)
    check_selection(L, idx, oracle.logit_error_bound(x, Wr, route_depth(wl.H, C)), wl.k)
    ref = oracle.latent_layer(wl, Wr, x[:1], Wd, Wu, g, idx=idx[:1],
                              routed_cache=_K3_WEIGHTS["routed"], shared_cache=_K3_WEIGHTS["shared"])
    assert _rms(ref["routed"]) > 0.1 * _rms(ref["shared"])
    assert_close(out[:1], ref["out"], f"latent K3 C={C} token 0")
    if C == 1:
        # gamma = 0 leaves the shared experts alone (the one-token kernels
        # that fold them into the dense launches)
        _, _, _, _, _, shared, _ = _run(wl, C, gamma_zero=True)
        assert_close(shared[:1], ref["shared"], "latent K3 C=1 shared part")


def test_latent_k3_one_token_repeat_bit_identical():
    """The one-token K3 latent layer gives bit-identical outputs on 12
    back-to-back calls over one workspace, and no bounded wait of the
    single-launch expert kernel expires."""
    R = rf()
    wl = synth.LATENT_WORKLOADS["k3_latent"]
    say("[latent] K3 shape C=1, 12 back-to-back calls")
    Wr, x, Wd, Wu, g = synth.latent_inputs(wl, 0, C=1)
    layer = R.LatentLayer(to_dev(Wr), _bits(Wd), to_dev(g), wl.eps, _bits(Wu),
                          cached_bank(wl.routed_bank()), cached_bank(wl.shared_bank()))
    ws = R.LatentWorkspace(layer, wl.k, 1)
    xd = to_dev(x)
    outs = [torch.empty((1, wl.H), dtype=torch.float32, device="cuda") for _ in range(12)]
    for o in outs:
        R.moe_latent_layer_fwd(layer, xd, 1, wl.k, o, None, None, ws)
    torch.cuda.synchronize()
    assert int(ws.tensor[4].item()) == 0
    first = outs[0].cpu().numpy().view(np.uint32)
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(o.cpu().numpy().view(np.uint32), first), f"call {i} differs"
