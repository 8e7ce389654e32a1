"""moe_layer_fwd_noalloc (the library's own device array as the workspace)
against moe_layer_fwd with a caller workspace, through the C ABI: two calls in
a row on each shape, the second with fewer tokens, outputs and selections
bit-identical (the same kernels run); the decode kernel's error word stays
clear; a call larger than the array is refused."""
import numpy as np
import pytest

import synth
from gpu_util import make_bank, say, to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import routed_expert_fp4_amd as rf
    rf.lib()
    torch.cuda.set_device(0)


def _both(rf, bank, wl, C, pool):
    Wr, x = synth.layer_inputs(wl, 0, C=C, pool=pool)
    Wr_d, x_d = to_dev(Wr), to_dev(x)
    res = []
    for noalloc in (False, True):
        out = torch.full((C, wl.H), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((C, wl.k), -1, dtype=torch.int32, device="cuda")
        w = torch.full((C, wl.k), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
            rf.moe_layer_fwd_noalloc(bank, Wr_d, x_d, C, wl.k, out, idx, w, err)
        else:
            ws = rf.Workspace(wl.E, wl.H, wl.I, wl.k, C)
            rf.moe_layer_fwd(bank, Wr_d, x_d, C, wl.k, out, idx, w, ws)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()))
        if noalloc:
            assert int(err.item()) == 0, "a bounded wait of the decode kernel expired"
    (o1, i1, w1), (o2, i2, w2) = res
    assert np.array_equal(i1, i2)
    assert np.array_equal(w1.view(np.uint32), w2.view(np.uint32))
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))


@pytest.mark.parametrize("name,Cs", [("w50_k16", (9, 1)), ("k3_stack", (4, 1)), ("tiny", (16, 3))])
def test_noalloc_matches_layer_fwd(name, Cs):
    import routed_expert_fp4_amd as rf
    wl = synth.WORKLOADS[name]
    bank = make_bank(wl.bank(0))
    for j, C in enumerate(Cs):
        say(f"[noalloc] {name} C={C}")
        _both(rf, bank, wl, C, pool=j + 1)
    del bank
    torch.cuda.empty_cache()


def test_noalloc_refuses_calls_beyond_its_array():
    import routed_expert_fp4_amd as rf
    wl = synth.WORKLOADS["k3_prefill"]
    C = 2048
    say(f"[noalloc] refused: K3 shape C={C}")
    assert rf.moe_workspace_size(wl.E, wl.H, wl.I, wl.k, C) > (40 << 20)
    bank = rf.Bank(wl.fmt, wl.E, wl.H, wl.I)            # contents never read
    out = torch.empty((C, wl.H), dtype=torch.float32, device="cuda")
    Wr = torch.zeros((wl.E, wl.H), dtype=torch.float32, device="cuda")
    x = torch.zeros((C, wl.H), dtype=torch.float32, device="cuda")
    with pytest.raises(rf.MoeError) as e:
        rf.moe_layer_fwd_noalloc(bank, Wr, x, C, wl.k, out)
    assert e.value.status == rf.MOE_ERR_WORKSPACE
    del bank
    torch.cuda.empty_cache()
