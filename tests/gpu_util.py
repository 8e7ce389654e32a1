"""Helpers shared by the GPU tests: banks filled on the device, inputs moved to
the device, and the parity rules (bit-exact routing with certified near-tie
handling, rel-L2 / max-abs tolerances on fp32 outputs)."""
from __future__ import annotations

import functools
import sys

import numpy as np

import oracle
import synth

RTOL_L2 = 2e-5          # ||gpu - ref||_2 / ||ref||_2
RTOL_MAX = 1e-4         # max|gpu - ref| / max|ref|


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_bank(spec: synth.BankSpec, device="cuda"):
    import torch
    import routed_expert_fp4_amd as rf
    import synth.device as sd
    bank = rf.Bank(spec.fmt, spec.num_experts, spec.hidden, spec.inter, device=device)
    sd.fill_bank(bank.storage.data_ptr(), bank.offsets, bank.stride, spec,
                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return bank


@functools.lru_cache(maxsize=4)
def cached_bank(spec: synth.BankSpec):
    return make_bank(spec)


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def route_depth(H: int, C: int = 1) -> int:
    """Upper bound on the rounding chain of the kernel's fp32 logit.  Up to 16
    tokens: each lane adds, per float4 of the row, a sum of 4 products (at most
    5 roundings) to its accumulator, for H/256 float4s or fewer; then a 6-level
    wave reduction and at most 4 split-K partials added in order (the decode
    kernel: half rows, then the two halves added).  More tokens: the
    matrix-core router, whose v_mfma_f32_16x16x4f32 adds its 4 products as 4
    chained FMAs (tests/test_gpu_fp4_mfma_model.py), accumulates each 32-wide
    K chunk on its own (32 roundings) and adds the H/32 chunk sums in order."""
    if C > 16:
        return 32 + H // 32 + 1
    return H // 32 + 16

# (test, tokens, near-tie tokens) of every selection check, reported at the end
# of the session (tests/conftest.py)
NEAR_TIES: list = []


def check_selection(L: np.ndarray, idx_gpu: np.ndarray, bound: np.ndarray, k: int,
                    steered: bool = False):
    """Per token: True if the GPU list equals the oracle's; otherwise the GPU
    list must be k distinct experts whose logits match the oracle's ranked
    logits position by position within the certified bound (a legitimate
    reordering of near-ties).  Returns the number of near-tie tokens, which
    is recorded for the session summary.  With steered (Zipf) routing the
    selected set sits far above the rest, so no near-tie may occur."""
    import os
    ref = oracle.topk(L, k)
    near = 0
    for t in range(L.shape[0]):
        g = idx_gpu[t]
        if np.array_equal(g, ref[t]):
            continue
        near += 1
        assert len(set(g.tolist())) == k, f"token {t}: duplicate experts {g}"
        for s in range(k):
            d = abs(L[t, g[s]] - L[t, ref[t, s]])
            assert d <= bound[t, g[s]] + bound[t, ref[t, s]], (
                f"token {t} slot {s}: gpu expert {g[s]} vs oracle {ref[t, s]}, gap {d}")
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    NEAR_TIES.append((test, int(L.shape[0]), near))
    if steered:
        assert near == 0, f"{near} near-tie tokens under steered routing"
    return near


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    r = oracle.rel_l2(got, ref)
    m = oracle.max_abs_ratio(got, ref)
    say(f"  {what}: rel_l2 {r:.3e}  max_abs/max|ref| {m:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert r <= RTOL_L2, f"{what}: rel_l2 {r:.3e} > {RTOL_L2}"
    assert m <= RTOL_MAX, f"{what}: max_abs ratio {m:.3e} > {RTOL_MAX}"
    return r, m
