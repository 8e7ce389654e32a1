"""The C-ABI library without a GPU: it loads, exports every function the header
declares, and rejects bad arguments on the host before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "routed_fp4.h")


@pytest.fixture(scope="module")
def rf():
    import routed_expert_fp4_amd as rf
    if not os.path.exists(rf.LIB_PATH):
        from routed_expert_fp4_amd import build
        build.build_library()
    rf.lib()
    return rf


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_]+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(rf):
    names = declared_functions()
    assert set(names) == set(rf.EXPORTS), names
    lib = ctypes.CDLL(rf.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(rf):
    assert rf.moe_version() == 1
    assert rf.status_string(0) == "ok"
    assert "workspace" in rf.status_string(-3)


def test_bank_layout(rf):
    off, stride = rf.moe_bank_layout(rf.MOE_FMT_NVFP4, 7168, 1536)
    sizes = [7168 * 1536 // 2] * 3 + [7168 * 1536 // 16] * 3 + [12]
    assert off[0] == 0
    for t in range(6):
        assert off[t + 1] >= off[t] + sizes[t] and off[t + 1] % 256 == 0
    assert stride % 4096 == 0 and stride >= off[6] + 12
    assert stride - (sum(sizes)) < 4096 + 7 * 256
    off, stride = rf.moe_bank_layout(rf.MOE_FMT_MXFP4, 3584, 3072)
    assert stride == 3 * 5_849_088     # sections already 4 KiB multiples
    with pytest.raises(rf.MoeError):
        rf.moe_bank_layout(3, 256, 128)
    with pytest.raises(rf.MoeError):
        rf.moe_bank_layout(rf.MOE_FMT_MXFP4, 250, 128)


def test_workspace_size(rf):
    n1 = rf.moe_workspace_size(896, 7168, 1536, 16, 1)
    n7 = rf.moe_workspace_size(896, 7168, 1536, 16, 7)
    assert 0 < n1 < n7 < 64 << 20
    assert rf.lib().moe_workspace_size(896, 7168, 1536, 16, 4097) == 0   # C too large
    n2048 = rf.moe_workspace_size(896, 7168, 1536, 16, 2048)               # prefill chunk
    assert 1.0e9 < n2048 < 1.4e9
    assert rf.lib().moe_workspace_size(896, 7168, 1536, 33, 1) == 0     # k too large
    assert rf.lib().moe_workspace_size(4, 256, 128, 5, 1) == 0          # k > E
    assert rf.lib().moe_workspace_size(2000, 256, 128, 5, 1) == 0       # E too large


def _bank(rf, **kw):
    off, stride = rf.moe_bank_layout(rf.MOE_FMT_MXFP4, 256, 128)
    b = rf.moe_bank(rf.MOE_FMT_MXFP4, 8, 256, 128, 0x10000, stride,
                    (ctypes.c_int64 * 7)(*off))
    for k, v in kw.items():
        setattr(b, k, v)
    return b


FAKE = ctypes.c_void_p(0x20000)   # never dereferenced: validation fails first


def test_layer_fwd_rejects_bad_arguments(rf):
    L = rf.lib()
    ws_n = rf.moe_workspace_size(8, 256, 128, 2, 4)

    def call(bank, x=FAKE, C=4, k=2, out=ctypes.c_void_p(0x30000), ws=FAKE, n=ws_n, wr=FAKE):
        return L.moe_layer_fwd(ctypes.byref(bank) if bank is not None else None, wr, x, C, k,
                               out, None, None, ws, n, None)

    assert call(None) == rf.MOE_ERR_INVALID_ARG
    assert call(_bank(rf, base=None)) == rf.MOE_ERR_INVALID_ARG
    assert call(_bank(rf, format=7)) == rf.MOE_ERR_UNSUPPORTED
    assert call(_bank(rf, hidden=250)) == rf.MOE_ERR_INVALID_ARG
    assert call(_bank(rf, num_experts=0)) == rf.MOE_ERR_UNSUPPORTED
    assert call(_bank(rf, expert_stride=1000)) == rf.MOE_ERR_INVALID_ARG
    assert call(_bank(rf, base=0x10008)) == rf.MOE_ERR_INVALID_ARG          # misaligned
    assert call(_bank(rf), x=None) == rf.MOE_ERR_INVALID_ARG
    assert call(_bank(rf), wr=None) == rf.MOE_ERR_INVALID_ARG
    assert call(_bank(rf), C=0) == rf.MOE_ERR_UNSUPPORTED
    assert call(_bank(rf), C=4097) == rf.MOE_ERR_UNSUPPORTED
    assert call(_bank(rf), C=17) == rf.MOE_ERR_WORKSPACE                    # sized for C=4
    assert call(_bank(rf), k=9) == rf.MOE_ERR_UNSUPPORTED                    # k > E
    assert call(_bank(rf), ws=None) == rf.MOE_ERR_WORKSPACE
    assert call(_bank(rf), n=ws_n - 1) == rf.MOE_ERR_WORKSPACE
    assert call(_bank(rf), out=FAKE) == rf.MOE_ERR_INVALID_ARG               # out aliases x


def test_route_and_expert_fwd_reject_bad_arguments(rf):
    L = rf.lib()
    n = rf.moe_workspace_size(8, 256, 32, 2, 4)
    assert L.moe_route(FAKE, FAKE, None, 4, 256, 8, 2, None, FAKE, FAKE, n, None) == rf.MOE_ERR_INVALID_ARG
    assert L.moe_route(None, None, None, 4, 256, 8, 2, FAKE, FAKE, FAKE, n, None) == rf.MOE_ERR_INVALID_ARG
    assert L.moe_route(FAKE, FAKE, None, 4, 250, 8, 2, FAKE, FAKE, FAKE, n, None) == rf.MOE_ERR_INVALID_ARG
    assert L.moe_route(FAKE, FAKE, None, 4, 256, 8, 0, FAKE, FAKE, FAKE, n, None) == rf.MOE_ERR_UNSUPPORTED
    assert L.moe_route(FAKE, FAKE, None, 4, 256, 8, 2, FAKE, FAKE, FAKE, 16, None) == rf.MOE_ERR_WORKSPACE
    b = _bank(rf)
    ws_n = rf.moe_workspace_size(8, 256, 128, 2, 4)
    assert L.moe_expert_fwd(ctypes.byref(b), FAKE, 4, 2, None, FAKE, ctypes.c_void_p(0x30000), FAKE, ws_n, None) == rf.MOE_ERR_INVALID_ARG
    assert L.moe_expert_fwd(ctypes.byref(b), FAKE, 4, 2, FAKE, FAKE, ctypes.c_void_p(0x30000), FAKE, 100, None) == rf.MOE_ERR_WORKSPACE
    assert L.moe_dequant(ctypes.byref(b), 8, 0, FAKE, None) == rf.MOE_ERR_INVALID_ARG
    assert L.moe_dequant(ctypes.byref(b), 0, 3, FAKE, None) == rf.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_init(None, 16, None) == rf.MOE_ERR_INVALID_ARG


def _mx_bank(rf, fmt=None, H=512, I=768, E=16):
    fmt = rf.MOE_FMT_MXFP4 if fmt is None else fmt
    off, stride = rf.moe_bank_layout(fmt, H, I)
    return rf.moe_bank(fmt, E, H, I, 0x100000, stride, (ctypes.c_int64 * 7)(*off))


def test_mx_mma_limits_and_rejections(rf):
    """Workspace sizing is pure host arithmetic; every rejected call returns
    before anything is enqueued."""
    L = rf.lib()
    b = _mx_bank(rf)
    size = L.moe_mx_mma_workspace_size(ctypes.byref(b), 4, 24, 2)
    assert size > 24 * 512 * 2                                   # at least x's two terms
    assert L.moe_mx_mma_workspace_size(ctypes.byref(b), 4, 24, 0) == 0
    assert L.moe_mx_mma_workspace_size(ctypes.byref(b), 4, 24, 7) == 0
    assert L.moe_mx_mma_workspace_size(ctypes.byref(b), 17, 24, 2) == 0       # k > E
    assert L.moe_mx_mma_workspace_size(ctypes.byref(b), 4, 0, 2) == 0
    assert L.moe_mx_mma_workspace_size(ctypes.byref(_mx_bank(rf, rf.MOE_FMT_NVFP4)), 4, 24, 2) == 0
    assert L.moe_mx_mma_workspace_size(ctypes.byref(_mx_bank(rf, H=384)), 4, 24, 2) == 0
    assert L.moe_mx_mma_workspace_size(None, 4, 24, 2) == 0
    out = ctypes.c_void_p(0x30000)
    ws = ctypes.c_void_p(0x400000)

    def call(bank=b, x=FAKE, o=out, ws=ws, n=size, terms=2, idx=FAKE):
        return L.moe_expert_fwd_mx_mma(ctypes.byref(bank) if bank is not None else None, x, 24, 4,
                                       idx, FAKE, o, terms, ws, n, None)

    assert call(bank=None) == rf.MOE_ERR_INVALID_ARG
    assert call(x=None) == rf.MOE_ERR_INVALID_ARG
    assert call(idx=None) == rf.MOE_ERR_INVALID_ARG
    assert call(o=FAKE) == rf.MOE_ERR_INVALID_ARG                           # out aliases x
    assert call(x=ctypes.c_void_p(0x20004)) == rf.MOE_ERR_INVALID_ARG       # misaligned x
    assert call(bank=_mx_bank(rf, rf.MOE_FMT_NVFP4)) == rf.MOE_ERR_UNSUPPORTED
    assert call(terms=0) == rf.MOE_ERR_UNSUPPORTED
    assert call(ws=None) == rf.MOE_ERR_WORKSPACE
    assert call(n=size - 1) == rf.MOE_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(0x400010)) == rf.MOE_ERR_WORKSPACE       # misaligned workspace


def test_latent_limits_and_rejections(rf):
    L = rf.lib()
    routed = _mx_bank(rf, rf.MOE_FMT_NVFP4, H=512, I=512, E=64)
    shared = _mx_bank(rf, rf.MOE_FMT_NVFP4, H=1024, I=1024, E=2)

    def layer(**kw):
        lay = rf.moe_latent_layer(1024, 0x20000, 0x40000, 0x50000, 1e-6, 0x60000, routed, shared)
        for k, v in kw.items():
            setattr(lay, k, v)
        return lay

    good = layer()
    size = L.moe_latent_workspace_size(ctypes.byref(good), 8, 4)
    assert size > 0
    assert L.moe_latent_workspace_size(None, 8, 4) == 0
    assert L.moe_latent_workspace_size(ctypes.byref(good), 8, 17) == 0       # C above the decode limit
    assert L.moe_latent_workspace_size(ctypes.byref(good), 65, 4) == 0       # k > E
    assert L.moe_latent_workspace_size(ctypes.byref(layer(w_down=None)), 8, 4) == 0
    assert L.moe_latent_workspace_size(ctypes.byref(layer(norm_eps=-1.0)), 8, 4) == 0
    assert L.moe_latent_workspace_size(ctypes.byref(layer(hidden=2048)), 8, 4) == 0   # shared bank width
    out = ctypes.c_void_p(0x30000)
    ws = ctypes.c_void_p(0x400000)

    def call(lay=good, x=ctypes.c_void_p(0x70000), o=out, C=4, ws=ws, n=size):
        return L.moe_latent_layer_fwd(ctypes.byref(lay) if lay is not None else None, x, C, 8, o,
                                      None, None, ws, n, None)

    assert call(lay=None) == rf.MOE_ERR_INVALID_ARG
    assert call(x=None) == rf.MOE_ERR_INVALID_ARG
    assert call(o=ctypes.c_void_p(0x70000)) == rf.MOE_ERR_INVALID_ARG       # out aliases x
    assert call(C=17) == rf.MOE_ERR_UNSUPPORTED
    assert call(ws=None) == rf.MOE_ERR_WORKSPACE
    assert call(n=size - 1) == rf.MOE_ERR_WORKSPACE
    assert call(x=ctypes.c_void_p(0x70004)) == rf.MOE_ERR_INVALID_ARG       # misaligned x
    assert call(lay=layer(w_up=0x60008)) == rf.MOE_ERR_INVALID_ARG          # misaligned routed_up
