"""Build and load the matrix-core and conversion rounding probes (test
infrastructure)."""
import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mfma_probe.hip")
LIB = os.path.join(HERE, "libmfmaprobe.so")


def build() -> str:
    tmp = LIB + ".tmp"
    subprocess.run(["/opt/rocm/bin/hipcc", "-O2", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", tmp],
                   check=True, capture_output=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is missing: run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    L.probe_mfma_f32.argtypes = [P, P, P, P, ctypes.c_int, P]
    L.probe_mfma_fp4.argtypes = [P, P, P, P, P, P, ctypes.c_int, P]
    L.probe_cvt_fp4_bf16.argtypes = [P, P, P, ctypes.c_int, P]
    L.probe_mfma_4x4_bf16.argtypes = [P, P, P, P, ctypes.c_int, P]
    for f in (L.probe_mfma_f32, L.probe_mfma_fp4, L.probe_cvt_fp4_bf16, L.probe_mfma_4x4_bf16):
        f.restype = ctypes.c_int
    return L
