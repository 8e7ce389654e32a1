"""Python binding of libroutedfp4 (the MI355X routed-expert FFN library).

Argument marshalling only: every step of the layer runs in the HIP kernels behind
the C ABI declared in ``include/routed_fp4.h``.  The functions carry the C names;
they take torch tensors that already live on the GPU, check dtype, shape, device
and contiguity, pass raw pointers and the current HIP stream, and raise
``MoeError`` on any non-OK status.  PyTorch is used for device memory and
streams only.

If the shared library has not been built this module raises on first use; there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libroutedfp4.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = 0, -1, -2, -3, -4
MOE_FMT_MXFP4, MOE_FMT_NVFP4 = 1, 2
MOE_NUM_TENSORS = 7
MOE_MAX_EXPERTS, MOE_MAX_TOPK, MOE_MAX_DECODE_TOKENS, MOE_MAX_TOKENS = 1024, 32, 16, 4096
BLOCK = {MOE_FMT_MXFP4: 32, MOE_FMT_NVFP4: 16}

EXPORTS = ("moe_version", "moe_status_string", "moe_bank_layout", "moe_workspace_size",
           "moe_workspace_init", "moe_route", "moe_expert_fwd", "moe_layer_fwd", "moe_dequant",
           "moe_latent_workspace_size", "moe_latent_layer_fwd", "moe_mx_mma_workspace_size",
           "moe_expert_fwd_mx_mma", "moe_layer_fwd_noalloc")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


class moe_bank(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("base", ctypes.c_void_p), ("expert_stride", ctypes.c_int64),
                ("offset", ctypes.c_int64 * MOE_NUM_TENSORS)]


class moe_latent_layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("w_router", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("norm_gamma", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float), ("w_up", ctypes.c_void_p),
                ("routed", moe_bank), ("shared", moe_bank)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() "
                               "(or routed_expert_fp4_amd.build.build_library()) first")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        sig = {
            "moe_version": ([], i32),
            "moe_status_string": ([i32], ctypes.c_char_p),
            "moe_bank_layout": ([i32, i32, i32, P, P], i32),
            "moe_workspace_size": ([i32, i32, i32, i32, i32], sz),
            "moe_workspace_init": ([P, sz, P], i32),
            "moe_route": ([P, P, P, i32, i32, i32, i32, P, P, P, sz, P], i32),
            "moe_expert_fwd": ([P, P, i32, i32, P, P, P, P, sz, P], i32),
            "moe_layer_fwd": ([P, P, P, i32, i32, P, P, P, P, sz, P], i32),
            "moe_dequant": ([P, i32, i32, P, P], i32),
            "moe_latent_workspace_size": ([P, i32, i32], sz),
            "moe_latent_layer_fwd": ([P, P, i32, i32, P, P, P, P, sz, P], i32),
            "moe_mx_mma_workspace_size": ([P, i32, i32, i32], sz),
            "moe_expert_fwd_mx_mma": ([P, P, i32, i32, P, P, P, i32, P, sz, P], i32),
            "moe_layer_fwd_noalloc": ([P, P, P, i32, i32, P, P, P, P, P], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t, dtype=None, shape=None, name="tensor"):
    """Device pointer of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------
# Bank layout and workspace
# ---------------------------------------------------------------------------
def moe_version() -> int:
    return lib().moe_version()


def moe_bank_layout(fmt: int, hidden: int, inter: int):
    """(offsets[7], expert_stride) of the library's preferred record layout."""
    off = (ctypes.c_int64 * MOE_NUM_TENSORS)()
    stride = ctypes.c_int64()
    _check("moe_bank_layout", lib().moe_bank_layout(fmt, hidden, inter, off, ctypes.byref(stride)))
    return list(off), stride.value


def moe_workspace_size(num_experts: int, hidden: int, inter: int, top_k: int, C: int) -> int:
    n = lib().moe_workspace_size(num_experts, hidden, inter, top_k, C)
    if n == 0:
        raise MoeError("moe_workspace_size", MOE_ERR_UNSUPPORTED)
    return n


def moe_workspace_init(ws, stream=None) -> None:
    _check("moe_workspace_init", lib().moe_workspace_init(_ptr(ws, name="ws"), ws.numel() * ws.element_size(), _stream(stream)))


class Bank:
    """An expert bank held in one device allocation, with its moe_bank struct."""

    def __init__(self, fmt: int, num_experts: int, hidden: int, inter: int, device="cuda",
                 storage=None):
        import torch
        self.fmt, self.E, self.H, self.I = fmt, num_experts, hidden, inter
        self.offsets, self.stride = moe_bank_layout(fmt, hidden, inter)
        nbytes = self.stride * num_experts
        self.storage = (torch.empty(nbytes, dtype=torch.uint8, device=device)
                        if storage is None else storage)
        if self.storage.numel() < nbytes:
            raise ValueError("bank storage too small")
        self.struct = moe_bank(fmt, num_experts, hidden, inter, self.storage.data_ptr(),
                               self.stride, (ctypes.c_int64 * MOE_NUM_TENSORS)(*self.offsets))

    def tensor_view(self, expert: int, tensor: int, nbytes: int):
        base = expert * self.stride + self.offsets[tensor]
        return self.storage[base: base + nbytes]


def _bank(b):
    return ctypes.byref(b.struct if isinstance(b, Bank) else b)


class Workspace:
    """A zero-initialised device workspace sized for (E, H, I, k, C)."""

    def __init__(self, num_experts, hidden, inter, top_k, C, device="cuda", stream=None):
        import torch
        n = moe_workspace_size(num_experts, hidden, inter, top_k, C)
        self.tensor = torch.empty((n + 255) // 256 * 256 // 4, dtype=torch.int32, device=device)
        moe_workspace_init(self.tensor, stream)

    @property
    def ptr(self):
        return ctypes.c_void_p(self.tensor.data_ptr())

    @property
    def nbytes(self):
        return self.tensor.numel() * 4


# ---------------------------------------------------------------------------
# The path
# ---------------------------------------------------------------------------
def moe_route(x, w_router, logits, C, H, E, k, topk_idx, topk_w, ws: Workspace, stream=None):
    """Router + top-k.  x None -> logits-in mode (logits is read)."""
    import torch
    _check("moe_route", lib().moe_route(
        _ptr(x, torch.float32, (C, H), "x"), _ptr(w_router, torch.float32, (E, H), "w_router"),
        _ptr(logits, torch.float32, (C, E), "logits"), C, H, E, k,
        _ptr(topk_idx, torch.int32, (C, k), "topk_idx"), _ptr(topk_w, torch.float32, (C, k), "topk_w"),
        ws.ptr, ws.nbytes, _stream(stream)))


def moe_expert_fwd(bank: Bank, x, C, k, topk_idx, topk_w, out, ws: Workspace, stream=None):
    import torch
    H = bank.H
    _check("moe_expert_fwd", lib().moe_expert_fwd(
        _bank(bank), _ptr(x, torch.float32, (C, H), "x"), C, k,
        _ptr(topk_idx, torch.int32, (C, k), "topk_idx"), _ptr(topk_w, torch.float32, (C, k), "topk_w"),
        _ptr(out, torch.float32, (C, H), "out"), ws.ptr, ws.nbytes, _stream(stream)))


def moe_layer_fwd(bank: Bank, w_router, x, C, k, out, topk_idx_out=None, topk_w_out=None,
                  ws: Workspace = None, stream=None):
    import torch
    H, E = bank.H, bank.E
    _check("moe_layer_fwd", lib().moe_layer_fwd(
        _bank(bank), _ptr(w_router, torch.float32, (E, H), "w_router"),
        _ptr(x, torch.float32, (C, H), "x"), C, k, _ptr(out, torch.float32, (C, H), "out"),
        _ptr(topk_idx_out, torch.int32, (C, k), "topk_idx_out"),
        _ptr(topk_w_out, torch.float32, (C, k), "topk_w_out"), ws.ptr, ws.nbytes, _stream(stream)))


def moe_layer_fwd_noalloc(bank: Bank, w_router, x, C, k, out, topk_idx_out=None,
                          topk_w_out=None, error_out=None, stream=None):
    """moe_layer_fwd on the library's own device array instead of a workspace."""
    import torch
    H, E = bank.H, bank.E
    _check("moe_layer_fwd_noalloc", lib().moe_layer_fwd_noalloc(
        _bank(bank), _ptr(w_router, torch.float32, (E, H), "w_router"),
        _ptr(x, torch.float32, (C, H), "x"), C, k, _ptr(out, torch.float32, (C, H), "out"),
        _ptr(topk_idx_out, torch.int32, (C, k), "topk_idx_out"),
        _ptr(topk_w_out, torch.float32, (C, k), "topk_w_out"),
        _ptr(error_out, torch.int32, (1,), "error_out"), _stream(stream)))


def moe_dequant(bank: Bank, expert: int, matrix: int, out, stream=None):
    import torch
    N, K = (bank.H, bank.I) if matrix == 2 else (bank.I, bank.H)
    _check("moe_dequant", lib().moe_dequant(_bank(bank), expert, matrix,
                                            _ptr(out, torch.float32, (N, K), "out"), _stream(stream)))


# ---------------------------------------------------------------------------
# Latent MoE layer (routed_down, routed experts, routed_norm, routed_up, shared)
# ---------------------------------------------------------------------------
class LatentLayer:
    """The device tensors of one latent MoE layer and its moe_latent_layer struct.
    w_router [E][H] fp32, w_down [L][H] and w_up [H][L] as int16/uint16 bf16
    bits, gamma [L] fp32; routed (hidden L) and shared (hidden H) are Banks."""

    def __init__(self, w_router, w_down, gamma, eps: float, w_up, routed: Bank, shared: Bank):
        import torch
        H, L = shared.H, routed.H
        _ptr(w_router, torch.float32, (routed.E, H), "w_router")
        if w_down.dtype not in (torch.int16, torch.uint16) or tuple(w_down.shape) != (L, H):
            raise ValueError(f"w_down must be bf16 bits of shape {(L, H)}")
        if w_up.dtype not in (torch.int16, torch.uint16) or tuple(w_up.shape) != (H, L):
            raise ValueError(f"w_up must be bf16 bits of shape {(H, L)}")
        _ptr(gamma, torch.float32, (L,), "gamma")
        self.keep = (w_router, w_down, gamma, w_up, routed, shared)
        self.H, self.L, self.E = H, L, routed.E
        self.struct = moe_latent_layer(H, w_router.data_ptr(), _ptr(w_down, name="w_down").value,
                                       gamma.data_ptr(), eps, _ptr(w_up, name="w_up").value,
                                       routed.struct, shared.struct)


class LatentWorkspace:
    def __init__(self, layer: LatentLayer, top_k: int, C: int, device="cuda", stream=None):
        import torch
        n = lib().moe_latent_workspace_size(ctypes.byref(layer.struct), top_k, C)
        if n == 0:
            raise MoeError("moe_latent_workspace_size", MOE_ERR_UNSUPPORTED)
        self.tensor = torch.empty((n + 255) // 256 * 256 // 4, dtype=torch.int32, device=device)
        moe_workspace_init(self.tensor, stream)

    @property
    def ptr(self):
        return ctypes.c_void_p(self.tensor.data_ptr())

    @property
    def nbytes(self):
        return self.tensor.numel() * 4


def moe_latent_layer_fwd(layer: LatentLayer, x, C, k, out, topk_idx_out=None, topk_w_out=None,
                         ws: LatentWorkspace = None, stream=None):
    import torch
    H = layer.H
    _check("moe_latent_layer_fwd", lib().moe_latent_layer_fwd(
        ctypes.byref(layer.struct), _ptr(x, torch.float32, (C, H), "x"), C, k,
        _ptr(out, torch.float32, (C, H), "out"),
        _ptr(topk_idx_out, torch.int32, (C, k), "topk_idx_out"),
        _ptr(topk_w_out, torch.float32, (C, k), "topk_w_out"), ws.ptr, ws.nbytes, _stream(stream)))


# ---------------------------------------------------------------------------
# MXFP4 experts on the block-scaled FP4 matrix cores
# ---------------------------------------------------------------------------
class MxMmaWorkspace:
    def __init__(self, bank: Bank, top_k: int, C: int, terms: int, device="cuda"):
        import torch
        n = lib().moe_mx_mma_workspace_size(_bank(bank), top_k, C, terms)
        if n == 0:
            raise MoeError("moe_mx_mma_workspace_size", MOE_ERR_UNSUPPORTED)
        self.tensor = torch.empty((n + 255) // 256 * 256 // 4, dtype=torch.int32, device=device)

    @property
    def ptr(self):
        return ctypes.c_void_p(self.tensor.data_ptr())

    @property
    def nbytes(self):
        return self.tensor.numel() * 4


def moe_expert_fwd_mx_mma(bank: Bank, x, C, k, topk_idx, topk_w, out, terms: int,
                          ws: MxMmaWorkspace, stream=None):
    import torch
    H = bank.H
    _check("moe_expert_fwd_mx_mma", lib().moe_expert_fwd_mx_mma(
        _bank(bank), _ptr(x, torch.float32, (C, H), "x"), C, k,
        _ptr(topk_idx, torch.int32, (C, k), "topk_idx"), _ptr(topk_w, torch.float32, (C, k), "topk_w"),
        _ptr(out, torch.float32, (C, H), "out"), terms, ws.ptr, ws.nbytes, _stream(stream)))
