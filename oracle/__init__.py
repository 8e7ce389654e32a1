"""CPU oracle of the routed-expert FFN -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``routed_expert_fp4_amd``)
never calls it and shares no code with it; the two meet only in the seeded
input generators of ``synth``.

The arithmetic lives in ``oracle.c`` (plain scalar C99, fp64 accumulation), which
``build()`` compiles with gcc.  This module loads it with ctypes and strings the
steps of one MoE layer together in the order the method defines them:

  router logits -> top-k by (logit desc, index asc) -> sigmoid weights
  renormalised over the k -> per selected expert: dequantise, gate/up mat-vecs,
  SwiGLU, down mat-vec -> weighted sum in slot order.

Sources: page "Kimi-K3 on 2x A40 -- measured findings", section "Why the placement
experiments all looked the same" (MUL_MAT_ID over the selected experts' matrices);
page "SparkInfer-K3", section "How the TP module works" (router, the chosen
top-16, the sum of the expert outputs); page "Kimi-K3 on the same pod, two
engines", section "Reason 1" (partial sums added in a fixed order).

The latent layer (``latent_layer``) adds, with numpy in fp64: routed_down and
routed_up as bf16 dense products, and the RMS norm of the routed sum (page
"SparkInfer-K3", sections "How the TP module works" and "Why the reduce is at
3584 and not 7168").  The shared experts reuse the expert FFN at weight 1.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against closed
forms, exact rational arithmetic, brute force and library routines.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, no FP contraction, OpenMP)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.run(["gcc", "-std=c99", "-O2", "-fno-fast-math", "-ffp-contract=off",
                        "-fopenmp", "-fPIC", "-shared", "-o", tmp, SRC, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i32, i64, f32, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        for name, args, res in [
            ("orc_e2m1", [i32], f64), ("orc_e8m0", [i32], f64), ("orc_e4m3", [i32], f64),
            ("orc_dequant_mx", [P, P, i64, i64, P], None),
            ("orc_dequant_nv", [P, P, f32, i64, i64, P], None),
            ("orc_router", [P, P, i32, i32, i32, P], None),
            ("orc_topk", [P, i32, i32, P], None),
            ("orc_topk_f32", [P, i32, i32, P], None),
            ("orc_route_weights", [P, i32, P], None),
            ("orc_silu", [f64], f64),
            ("orc_expert_ffn", [P, P, P, P, i32, i32, P], None),
            ("orc_expert_hidden", [P, P, P, i32, i32, P], None),
            ("orc_combine", [P, P, i32, i32, P], None),
            ("orc_threads", [], i32), ("orc_set_threads", [i32], None),
        ]:
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# Scalar encodings
# ---------------------------------------------------------------------------
def e2m1(code: int) -> float:
    return lib().orc_e2m1(code)


def e8m0(byte: int) -> float:
    return lib().orc_e8m0(byte)


def e4m3(byte: int) -> float:
    return lib().orc_e4m3(byte)


def silu(z: float) -> float:
    return lib().orc_silu(z)


# ---------------------------------------------------------------------------
# Dequantisation
# ---------------------------------------------------------------------------
def dequant(fmt: int, codes: np.ndarray, scales: np.ndarray, g: float = 1.0) -> np.ndarray:
    """codes [N][K/2] uint8, scales [N][K/B] uint8 -> fp32 [N][K]."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    N, K = codes.shape[0], codes.shape[1] * 2
    out = np.empty((N, K), np.float32)
    if fmt == synth.FMT_MX:
        assert scales.shape == (N, K // 32)
        lib().orc_dequant_mx(_p(codes), _p(scales), N, K, _p(out))
    else:
        assert scales.shape == (N, K // 16)
        lib().orc_dequant_nv(_p(codes), _p(scales), float(g), N, K, _p(out))
    return out


def expert_weights(spec: synth.BankSpec, expert: int):
    """(Wg [I][H], Wu [I][H], Wd [H][I]) fp32, dequantised from the host
    regeneration of the expert's bytes."""
    t = synth.expert_tensors(spec, expert)
    g = t["globals"]
    Wg = dequant(spec.fmt, t["gate_codes"], t["gate_scales"], g[0])
    Wu = dequant(spec.fmt, t["up_codes"], t["up_scales"], g[1])
    Wd = dequant(spec.fmt, t["down_codes"], t["down_scales"], g[2])
    return Wg, Wu, Wd


# ---------------------------------------------------------------------------
# Routing
# ---------------------------------------------------------------------------
def router_logits(x: np.ndarray, Wr: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    Wr = np.ascontiguousarray(Wr, np.float32)
    C, H = x.shape
    E = Wr.shape[0]
    out = np.empty((C, E), np.float64)
    lib().orc_router(_p(x), _p(Wr), C, H, E, _p(out))
    return out


def topk(values: np.ndarray, k: int) -> np.ndarray:
    """Row-wise top-k by (value desc, index asc); fp32 rows select on fp32."""
    v = np.atleast_2d(values)
    out = np.empty((v.shape[0], k), np.int32)
    for t in range(v.shape[0]):
        row = np.ascontiguousarray(v[t])
        if row.dtype == np.float32:
            lib().orc_topk_f32(_p(row), row.shape[0], k, _p(out[t]))
        else:
            row = row.astype(np.float64)
            lib().orc_topk(_p(row), row.shape[0], k, _p(out[t]))
    return out


def route_weights(l_sel: np.ndarray) -> np.ndarray:
    l_sel = np.ascontiguousarray(l_sel, np.float64)
    w = np.empty_like(l_sel)
    lib().orc_route_weights(_p(l_sel), l_sel.shape[0], _p(w))
    return w


def route(x: np.ndarray, Wr: np.ndarray, k: int):
    """(logits fp64 [C][E], idx [C][k], w fp64 [C][k])."""
    L = router_logits(x, Wr)
    idx = topk(L, k)
    w = np.stack([route_weights(L[t, idx[t]]) for t in range(L.shape[0])])
    return L, idx, w


# ---------------------------------------------------------------------------
# Experts and the whole layer
# ---------------------------------------------------------------------------
def expert_ffn(Wg, Wu, Wd, x: np.ndarray) -> np.ndarray:
    I, H = Wg.shape
    x = np.ascontiguousarray(x, np.float32)
    y = np.empty(H, np.float64)
    lib().orc_expert_ffn(_p(Wg), _p(Wu), _p(Wd), _p(x), H, I, _p(y))
    return y


def expert_hidden(Wg, Wu, x: np.ndarray) -> np.ndarray:
    I, H = Wg.shape
    x = np.ascontiguousarray(x, np.float32)
    h = np.empty(I, np.float64)
    lib().orc_expert_hidden(_p(Wg), _p(Wu), _p(x), H, I, _p(h))
    return h


def combine(w: np.ndarray, ys: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w, np.float64)
    ys = np.ascontiguousarray(ys, np.float64)
    k, H = ys.shape
    out = np.empty(H, np.float64)
    lib().orc_combine(_p(w), _p(ys), k, H, _p(out))
    return out


def experts_forward(spec: synth.BankSpec, x: np.ndarray, idx: np.ndarray,
                    w: np.ndarray, weights_cache: dict | None = None) -> np.ndarray:
    """out [C][H] fp64 for a given selection (idx [C][k], w [C][k]).
    Each distinct expert is dequantised once."""
    C, H = x.shape
    k = idx.shape[1]
    cache = {} if weights_cache is None else weights_cache
    out = np.empty((C, H), np.float64)
    for t in range(C):
        ys = np.empty((k, H), np.float64)
        for s in range(k):
            e = int(idx[t, s])
            if e not in cache:
                cache[e] = expert_weights(spec, e)
            ys[s] = expert_ffn(*cache[e], x[t])
        out[t] = combine(w[t], ys)
    return out


def layer(spec: synth.BankSpec, Wr: np.ndarray, x: np.ndarray, k: int,
          idx: np.ndarray | None = None):
    """One MoE layer.  With ``idx`` given, that selection is evaluated instead of
    the oracle's own (the weights are still the oracle's sigmoid-renormalised
    ones for that selection)."""
    L = router_logits(x, Wr)
    if idx is None:
        idx = topk(L, k)
    idx = np.asarray(idx, np.int32)
    w = np.stack([route_weights(L[t, idx[t]]) for t in range(L.shape[0])])
    out = experts_forward(spec, x, idx, w)
    return {"logits": L, "idx": idx, "w": w, "out": out}


# ---------------------------------------------------------------------------
# Latent MoE layer
# ---------------------------------------------------------------------------
# Page "SparkInfer-K3", section "How the TP module works": the router, routed_down
# (hidden to latent) and the routed experts form the partial phase; routed_norm,
# routed_up (latent to hidden) and the shared experts form the finish phase.
# Section "Why the reduce is at 3584 and not 7168": the RMS norm acts on the
# sum of the routed experts' outputs.  Section "The model": 2 shared experts,
# latent width 3584, expert FFN 3072.  The shared experts see the hidden x and
# enter with weight 1 each (the pages give them no gate).
def bf16_matrix(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> their exact values in fp64."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def dense(W_bits: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y [C][N] = x [C][K] times W^T for a bf16 matrix W [N][K], in fp64."""
    return np.asarray(x, np.float64) @ bf16_matrix(W_bits).T


def rms_norm(y: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """gamma * y / sqrt(mean(y^2) + eps), row by row, in fp64."""
    y = np.asarray(y, np.float64)
    ms = np.mean(y * y, axis=-1, keepdims=True)
    return np.asarray(gamma, np.float64) * y / np.sqrt(ms + float(eps))


def latent_layer(wl: synth.LatentWorkload, Wr: np.ndarray, x: np.ndarray, Wd_bits: np.ndarray,
                 Wu_bits: np.ndarray, gamma: np.ndarray, idx: np.ndarray | None = None,
                 layer: int = 0, routed_cache: dict | None = None,
                 shared_cache: dict | None = None):
    """One latent MoE layer for x [C][H].  With ``idx`` given, that routed
    selection is evaluated (weights still the oracle's for it).  The routed
    experts take x_lat as fp32, as every expert input is."""
    C = x.shape[0]
    L = router_logits(x, Wr)
    if idx is None:
        idx = topk(L, wl.k)
    idx = np.asarray(idx, np.int32)
    w = np.stack([route_weights(L[t, idx[t]]) for t in range(C)])
    xlat = dense(Wd_bits, x)
    ylat = experts_forward(wl.routed_bank(layer), xlat.astype(np.float32), idx, w, routed_cache)
    yn = rms_norm(ylat, gamma, wl.eps)
    routed = dense(Wu_bits, yn)
    sidx = np.tile(np.arange(wl.n_shared, dtype=np.int32), (C, 1))
    shared = experts_forward(wl.shared_bank(layer), x, sidx, np.ones((C, wl.n_shared)),
                             shared_cache)
    return {"logits": L, "idx": idx, "w": w, "xlat": xlat, "ylat": ylat, "routed": routed,
            "shared": shared, "out": routed + shared}


# ---------------------------------------------------------------------------
# Comparison helpers
# ---------------------------------------------------------------------------
def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, np.float64)
    d = np.asarray(got, np.float64) - ref
    n = math.sqrt(float(np.sum(ref * ref)))
    return math.sqrt(float(np.sum(d * d))) / n if n > 0 else math.sqrt(float(np.sum(d * d)))


def max_abs_ratio(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / max|ref|."""
    ref = np.asarray(ref, np.float64)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    d = float(np.max(np.abs(np.asarray(got, np.float64) - ref))) if ref.size else 0.0
    return d / m if m > 0 else d


def logit_error_bound(x: np.ndarray, Wr: np.ndarray, depth: int) -> np.ndarray:
    """Certified bound on |fp32 logit - exact logit| for a summation whose
    longest chain of roundings has ``depth`` steps (Higham, Accuracy and
    Stability of Numerical Algorithms, 2nd ed., section 3.1: |error| <=
    gamma_depth * sum|x_h W_eh|, gamma_n = n u / (1 - n u), u = 2^-24).
    Returns [C][E]."""
    u = 2.0 ** -24
    gamma = depth * u / (1.0 - depth * u)
    a = np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(Wr, np.float64)).T
    return gamma * a + 2.0 ** -149
