"""Device-side fill of synthetic expert banks (input generation only), and the
bench's read-bandwidth calibration.

``fill_bank`` writes every tensor of every expert of a bank with the same
counter-based bytes that ``synth.expert_tensor_bytes`` regenerates on the host.
Where the tensors sit inside an expert record (offsets, stride) is given by the
caller, so this module knows nothing of any kernel's layout choices.
``stream_read`` is a plain streaming read, the yardstick for the achievable
HBM read rate that bench.py reports beside the 8 TB/s peak.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

from . import BankSpec, FMT_NV

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fill.hip")
LIB = os.path.join(HERE, "libsynthfill.so")
_lib = None


def build(force: bool = False) -> str:
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "-O3", "-std=c++17", "-fPIC",
               "-shared", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", SRC, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {SRC}:\n{r.stderr}")
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is missing: build it with synth.device.build()")
        L = ctypes.CDLL(LIB)
        L.synth_fill_tensor.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_uint64, ctypes.c_int32,
                                        ctypes.c_void_p]
        L.synth_fill_tensor.restype = ctypes.c_int
        L.synth_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p]
        L.synth_stream_read.restype = ctypes.c_int
        _lib = L
    return _lib


def fill_bank(ptr: int, offsets, stride: int, spec: BankSpec, stream_handle: int = 0) -> None:
    """Fill experts [0, spec.num_experts) of the bank at device address ``ptr``;
    tensor t of expert e starts at ptr + e*stride + offsets[t]."""
    for t in range(7):
        nbytes = spec.tensor_bytes(t)
        if nbytes == 0:
            continue
        rc = lib().synth_fill_tensor(ctypes.c_void_p(ptr), stride, spec.num_experts,
                                     offsets[t], nbytes, t, spec.fmt, spec.seed, spec.layer,
                                     ctypes.c_void_p(stream_handle))
        if rc != 0:
            raise RuntimeError(f"synth_fill_tensor(tensor {t}) returned {rc}")


def stream_read(ptr: int, nbytes: int, blocks: int, sink_ptr: int, stream_handle: int = 0) -> None:
    """The bench's read-bandwidth calibration: a plain streaming read of
    nbytes at device address ``ptr`` (not part of the method)."""
    rc = lib().synth_stream_read(ctypes.c_void_p(ptr), nbytes, blocks, ctypes.c_void_p(sink_ptr),
                                 ctypes.c_void_p(stream_handle))
    if rc != 0:
        raise RuntimeError(f"synth_stream_read returned {rc}")
