"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module draws inputs only.  It holds none of the method's arithmetic: no
dequantisation, no mat-vec, no routing decision.  Two kinds of input exist.

* Small fp32 tensors (the router matrix ``W_r``, the activations ``x``) are drawn
  with numpy's PCG64 from a ``SeedSequence([seed, layer, stream])`` and copied to
  the device by whoever needs them there.

* Expert weight banks (up to ~200 GB) cannot be drawn on the host, so every byte
  is a pure function of ``(seed, layer, expert, tensor, index)``: a counter-based
  generator built on the SplitMix64 output function (G. Steele, D. Lea,
  C. Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014).
  ``fill.hip`` fills a device bank from the same definition, and
  ``expert_tensor_bytes`` regenerates any one expert's tensors on the host, so the
  oracle's inputs never come from the device.  Tests byte-compare the two.

Weight formats follow the workloads the pages name for the routed experts: a
4-bit e2m1 code per element with one e8m0 scale per 32 elements (MXFP4, page
"Kimi-K3 on 2x A40 -- measured findings", section "Why the placement experiments
all looked the same", the MUL_MAT_ID microbenchmark), or e2m1 codes with one
fp8-e4m3 scale per 16 elements plus an fp32 scale per tensor (NVFP4, page
"Kimi-K3 on the same pod, two engines", section "Same hardware, same weights").
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# ----------------------------------------------------------------------------
# Counter-based byte generator
# ----------------------------------------------------------------------------
GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

# Tensor ids inside one expert.  The same ids key the device fill.
T_GATE_CODES, T_UP_CODES, T_DOWN_CODES = 0, 1, 2
T_GATE_SCALES, T_UP_SCALES, T_DOWN_SCALES = 3, 4, 5
T_GLOBALS = 6
TENSOR_NAMES = ("gate_codes", "up_codes", "down_codes",
                "gate_scales", "up_scales", "down_scales", "globals")

FMT_MX, FMT_NV = 1, 2          # same numbering as the C-ABI's format enum
BLOCK = {FMT_MX: 32, FMT_NV: 16}


def _mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (mod 2^64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (numpy wraps mod 2^64)."""
    z = z.astype(np.uint64, copy=True)
    z ^= z >> np.uint64(30)
    z *= np.uint64(MIX1)
    z ^= z >> np.uint64(27)
    z *= np.uint64(MIX2)
    z ^= z >> np.uint64(31)
    return z


def stream_key(seed: int, layer: int, expert: int, tensor: int) -> int:
    """64-bit key of one tensor's byte stream: chained SplitMix64 mixing."""
    seed, layer, expert, tensor = int(seed), int(layer), int(expert), int(tensor)
    k = _mix64_int(seed + GAMMA)
    k = _mix64_int(k ^ (layer + GAMMA))
    k = _mix64_int(k ^ (expert + 2 * GAMMA))
    k = _mix64_int(k ^ (tensor + 3 * GAMMA))
    return k


def stream_words(key: int, start: int, count: int) -> np.ndarray:
    """Words ``start .. start+count-1`` of a stream: mix64(key + (i+1)*GAMMA)."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    return _mix64_np(np.uint64(key) + i * np.uint64(GAMMA))


# ----------------------------------------------------------------------------
# Bank description (logical tensors; the device layout is the library's)
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class BankSpec:
    fmt: int          # FMT_MX or FMT_NV
    num_experts: int
    hidden: int       # H: K of gate/up, N of down
    inter: int        # I: N of gate/up, K of down
    seed: int = 0
    layer: int = 0

    @property
    def block(self) -> int:
        return BLOCK[self.fmt]

    def tensor_shape(self, tensor: int) -> tuple[int, int]:
        """(rows, bytes per row) of one logical tensor of one expert."""
        H, I, B = self.hidden, self.inter, self.block
        return {
            T_GATE_CODES: (I, H // 2), T_UP_CODES: (I, H // 2),
            T_DOWN_CODES: (H, I // 2),
            T_GATE_SCALES: (I, H // B), T_UP_SCALES: (I, H // B),
            T_DOWN_SCALES: (H, I // B),
            T_GLOBALS: (1, 12 if self.fmt == FMT_NV else 0),
        }[tensor]

    def tensor_bytes(self, tensor: int) -> int:
        r, c = self.tensor_shape(tensor)
        return r * c

    def expert_bytes(self) -> int:
        """Bytes one expert's weights occupy (codes + scales + globals)."""
        return sum(self.tensor_bytes(t) for t in range(7))


def _scale_byte(fmt: int, w: np.ndarray) -> np.ndarray:
    if fmt == FMT_MX:
        # e8m0 exponent uniform on {-4..0}: bytes 123..127
        return (np.uint64(127) - (w % np.uint64(5))).astype(np.uint8)
    # e4m3 normal values 0.0625 .. 0.9375: bytes 0x18 .. 0x37
    return (np.uint64(0x18) + (w % np.uint64(32))).astype(np.uint8)


def expert_tensor_bytes(spec: BankSpec, expert: int, tensor: int) -> np.ndarray:
    """Host regeneration of one tensor of one expert, as a [rows][bytes] uint8 array.

    Codes: byte j is byte (j mod 8) of word (j div 8), little endian.
    Scales: byte j comes from word j (MX: 127 - w mod 5; NV: 0x18 + w mod 32).
    Globals (NV): three fp32 values 1 + (w_m >> 41) * 2^-23, m = gate, up, down.
    """
    rows, cols = spec.tensor_shape(tensor)
    key = stream_key(spec.seed, spec.layer, expert, tensor)
    n = rows * cols
    if tensor in (T_GATE_CODES, T_UP_CODES, T_DOWN_CODES):
        w = stream_words(key, 0, n // 8)
        return w.astype("<u8").view(np.uint8).reshape(rows, cols)
    if tensor in (T_GATE_SCALES, T_UP_SCALES, T_DOWN_SCALES):
        return _scale_byte(spec.fmt, stream_words(key, 0, n)).reshape(rows, cols)
    if spec.fmt != FMT_NV:
        return np.zeros((1, 0), np.uint8)
    return global_scales(spec, expert).view(np.uint8).reshape(1, 12)


def global_scales(spec: BankSpec, expert: int) -> np.ndarray:
    """The three per-tensor fp32 scales (gate, up, down) of an NV expert."""
    key = stream_key(spec.seed, spec.layer, expert, T_GLOBALS)
    w = stream_words(key, 0, 3)
    m = (w >> np.uint64(41)).astype(np.float64)
    return (1.0 + m * 2.0 ** -23).astype("<f4")


def expert_tensors(spec: BankSpec, expert: int) -> dict:
    """All named tensors of one expert (codes and scales as uint8 [rows][cols])."""
    out = {TENSOR_NAMES[t]: expert_tensor_bytes(spec, expert, t) for t in range(6)}
    out["globals"] = (global_scales(spec, expert) if spec.fmt == FMT_NV
                      else np.ones(3, np.float32))
    return out


# ----------------------------------------------------------------------------
# Small fp32 tensors
# ----------------------------------------------------------------------------
S_ROUTER, S_X, S_ROUTING = 0, 1, 2


def rng_for(seed: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, layer, stream]))


def router_weights(seed: int, layer: int, E: int, H: int, std: float = 0.02) -> np.ndarray:
    """W_r [E][H] fp32, entries N(0, std^2)."""
    g = rng_for(seed, layer, S_ROUTER)
    return (g.standard_normal((E, H), dtype=np.float32) * np.float32(std))


def activations(seed: int, layer: int, C: int, H: int, pool: int = 0) -> np.ndarray:
    """x [C][H] fp32, entries N(0,1).  ``pool`` selects an independent draw."""
    g = np.random.default_rng(np.random.SeedSequence([seed, layer, S_X, pool]))
    return g.standard_normal((C, H), dtype=np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even), returned as fp32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32)


def zipf_sets(seed: int, layer: int, C: int, E: int, k: int, s: float,
              pool: int = 0) -> np.ndarray:
    """Per token, k distinct experts drawn without replacement with
    P(rank r) proportional to r^-s over one seeded permutation of the experts
    (Gumbel-top-k: the k largest of log p + Gumbel noise).  Returns [C][k] int32."""
    g = np.random.default_rng(np.random.SeedSequence([seed, layer, S_ROUTING]))
    perm = g.permutation(E)                       # expert holding rank r
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    gt = np.random.default_rng(np.random.SeedSequence([seed, layer, S_ROUTING, pool]))
    out = np.empty((C, k), np.int32)
    for t in range(C):
        keys = logp + gt.gumbel(size=E)
        ranks = np.argsort(-keys, kind="stable")[:k]
        out[t] = perm[ranks]
    return out


def steer(z: np.ndarray, Wr: np.ndarray, sets: np.ndarray, alpha: float) -> np.ndarray:
    """Activations that make the router prefer a chosen expert set:
    x_t = z_t + alpha * sum_{e in S_t} W_r[e] / |W_r[e]|^2  (fp32 result)."""
    W = Wr.astype(np.float64)
    dirs = W / np.sum(W * W, axis=1, keepdims=True)
    x = z.astype(np.float64).copy()
    for t in range(z.shape[0]):
        x[t] += alpha * dirs[sets[t]].sum(axis=0)
    return x.astype(np.float32)


def steer_alpha(H: int, std: float = 0.02) -> float:
    """Steering strength: 10 standard deviations of a natural logit."""
    return 10.0 * std * math.sqrt(H)


# ----------------------------------------------------------------------------
# The workloads (shapes, formats, distributions)
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    fmt: int
    E: int
    k: int
    H: int
    I: int
    C: int
    layers: int = 1
    routing: str = "natural"   # "natural" or "zipf"
    zipf_s: float = 0.0
    bf16_x: bool = False
    seed: int = 0

    def bank(self, layer: int = 0) -> BankSpec:
        return BankSpec(self.fmt, self.E, self.H, self.I, self.seed, layer)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", FMT_MX, 8, 2, 256, 128, 4),
    "w50_k16": Workload("w50_k16", FMT_MX, 448, 16, 3584, 3072, 1),
    "w50_k8": Workload("w50_k8", FMT_MX, 448, 8, 3584, 3072, 1),
    "w50_c7_k8": Workload("w50_c7_k8", FMT_MX, 448, 8, 3584, 3072, 7, 1, "zipf", 1.1),
    "w50_c7_k16": Workload("w50_c7_k16", FMT_MX, 448, 16, 3584, 3072, 7, 1, "zipf", 1.1),
    "k3_stack": Workload("k3_stack", FMT_NV, 896, 16, 7168, 1536, 1, 12),
    "k3_stack_zipf": Workload("k3_stack_zipf", FMT_NV, 896, 16, 7168, 1536, 1, 12, "zipf", 1.2),
    "k3_prefill": Workload("k3_prefill", FMT_NV, 896, 16, 7168, 1536, 2048, 1, "zipf", 1.0, True),
    # a 2048-token chunk through one MXFP4 layer of the W50 shape (the format the
    # block-scaled FP4 matrix cores take as stored)
    "w50_prefill": Workload("w50_prefill", FMT_MX, 448, 8, 3584, 3072, 2048, 1, "zipf", 1.0, True),
}


# ----------------------------------------------------------------------------
# Latent MoE layer (routed_down, routed experts, routed_norm, routed_up, shared)
# ----------------------------------------------------------------------------
S_DOWN, S_UP, S_GAMMA = 11, 12, 13


def dense_bf16(seed: int, layer: int, stream: int, N: int, K: int) -> np.ndarray:
    """A dense [N][K] matrix of N(0, 1/K) entries rounded to bf16, as uint16 bits."""
    g = rng_for(seed, layer, stream)
    a = g.standard_normal((N, K), dtype=np.float32) * np.float32(1.0 / math.sqrt(K))
    return (round_to_bf16(a).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class LatentWorkload:
    """A latent MoE layer: router on the hidden x (H), routed experts in the
    latent space (L, FFN I), n_shared shared experts on x (H, FFN I_shared).
    The norm's gamma is gamma_scale * (1 + 0.1 N(0, 1)): the synthetic banks'
    expert outputs are large, and gamma_scale (a power of two near the shared
    part's RMS) brings the normalised routed part to the same size, as a
    trained norm weight would."""
    name: str
    fmt: int
    E: int
    k: int
    H: int
    L: int
    I: int
    n_shared: int
    I_shared: int
    C: int
    layers: int = 1
    eps: float = 1e-6
    gamma_scale: float = 1.0
    seed: int = 0

    def routed_bank(self, layer: int = 0) -> BankSpec:
        return BankSpec(self.fmt, self.E, self.L, self.I, self.seed, layer)

    def shared_bank(self, layer: int = 0) -> BankSpec:
        return BankSpec(self.fmt, self.n_shared, self.H, self.I_shared, self.seed + 1, layer)

    def with_(self, **kw) -> "LatentWorkload":
        return dataclasses.replace(self, **kw)


LATENT_WORKLOADS = {
    # page "SparkInfer-K3", section "The model": 896 routed experts, top-16,
    # 2 shared, latent 3584, expert FFN 3072, hidden 7168
    "k3_latent": LatentWorkload("k3_latent", FMT_NV, 896, 16, 7168, 3584, 3072, 2, 3072, 1, 4,
                                gamma_scale=2.0 ** 20),
}


def latent_inputs(w: LatentWorkload, layer: int, pool: int = 0, C: int | None = None):
    """(W_r [E][H] fp32, x [C][H] fp32, W_down [L][H] bf16 bits, W_up [H][L]
    bf16 bits, gamma [L] fp32) of one latent layer."""
    C = w.C if C is None else C
    Wr = router_weights(w.seed, layer, w.E, w.H)
    x = activations(w.seed, layer, C, w.H, pool)
    Wd = dense_bf16(w.seed, layer, S_DOWN, w.L, w.H)
    Wu = dense_bf16(w.seed, layer, S_UP, w.H, w.L)
    g = rng_for(w.seed, layer, S_GAMMA)
    gamma = (w.gamma_scale * (1.0 + 0.1 * g.standard_normal(w.L))).astype(np.float32)
    return Wr, x, Wd, Wu, gamma


def layer_inputs(w: Workload, layer: int, pool: int = 0, C: int | None = None):
    """(W_r, x) of one layer of a workload; x steered for Zipf routing and
    rounded to bf16 when the workload says so."""
    C = w.C if C is None else C
    Wr = router_weights(w.seed, layer, w.E, w.H)
    x = activations(w.seed, layer, C, w.H, pool)
    if w.routing == "zipf":
        sets = zipf_sets(w.seed, layer, C, w.E, w.k, w.zipf_s, pool)
        x = steer(x, Wr, sets, steer_alpha(w.H))
    if w.bf16_x:
        x = round_to_bf16(x)
    return Wr, x
