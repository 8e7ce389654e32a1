"""Build step for libroutedfp4.so (hipcc, gfx950).

Packed-fp32 instructions are disabled (``-packed-fp32-ops``); the float code is
ordinary scalar fp32.  The library is built in-tree next to this file.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", "routed_fp4.hip"), os.path.join(HERE, "csrc", "batched.hip"),
        os.path.join(HERE, "csrc", "latent.hip"), os.path.join(HERE, "csrc", "mxmma.hip"),
        os.path.join(HERE, "csrc", "noalloc.hip")]
OUT = os.path.join(HERE, "libroutedfp4.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc(srcs, out: str, extra=()) -> str:
    srcs = [srcs] if isinstance(srcs, str) else list(srcs)
    tmp = out + ".tmp"
    cmd = [HIPCC, *HIP_FLAGS, f"-I{INCLUDE}", *extra, *srcs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {srcs}:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build_library() -> str:
    """Compile the HIP kernels and the C ABI into libroutedfp4.so: one object
    per source, compiled in parallel, then linked."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = [f for f in HIP_FLAGS if f != "-shared"]

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        tmp = obj + ".tmp"
        r = subprocess.run([HIPCC, *flags, f"-I{INCLUDE}", "-c", src, "-o", tmp],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        os.replace(tmp, obj)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SRCS), 8)) as ex:
        objs = list(ex.map(compile_one, SRCS))
    tmp = OUT + ".tmp"
    r = subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT
