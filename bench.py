"""Decode benchmark of the routed-expert FFN on one MI355X.

Workload (default): a stack of 12 MoE layers, each 896 experts, top-16,
hidden 7168, intermediate 1536, NVFP4-style weights (~18.58 MB per expert, the
whole 199.8 GB bank resident in HBM), batch 1 token, router logits from the
natural router (uniform routing).  One step = one token through the 12 layers,
12 dependent moe_layer_fwd calls on one stream.  Each step takes the next of
16 pre-drawn tokens per layer, so consecutive steps select different experts.

Prints one JSON line: the metric (MoE-layer decode us/token, with achieved HBM
GB/s on selected-expert bytes), a roofline object for the kernel that runs the
whole layer for one token (k_moe1: one launch per moe_layer_fwd call; its
algorithmic bytes are the router weights plus the selected experts' weights,
timed with HIP events on the stream it is launched on) and the CPU oracle timed
on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer decode µs/token + achieved HBM GB/s (% of peak), 896 experts top-16"
HBM_PEAK_GBPS = 8000.0
POOL = 16            # pre-drawn inputs per layer (2 for prefill-sized calls)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="k3_stack",
                   choices=["k3_stack", "k3_stack_zipf", "w50_k16", "w50_k8", "w50_c7_k8",
                            "w50_c7_k16", "tiny", "k3_prefill", "w50_prefill", "k3_latent"],
                   help="k3_stack (the headline: 12 layers, uniform routing), k3_stack_zipf "
                        "(Zipf s=1.2), one of the single-layer decode workloads, or k3_latent "
                        "(whole latent layers: router, routed_down, routed experts, norm, "
                        "routed_up, shared experts)")
    p.add_argument("--tokens", type=int, default=0,
                   help="tokens per call instead of the workload's own (a sweep over C reuses "
                        "one workload's bank, routing and shapes)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-read-calibration", action="store_true",
                   help="skip measuring the achievable read rate beside the result")
    p.add_argument("--cpu-layers", type=int, default=1,
                   help="layer-tokens of the workload the CPU oracle is timed on")
    p.add_argument("--layer-only", action="store_true",
                   help="time only the whole-layer step (no expert-only / route-only loops), "
                        "so a kernel trace holds only the layer kernel's launches")
    p.add_argument("--mx-mma", type=int, default=0, metavar="T",
                   help="MXFP4 workloads: run the experts on the block-scaled FP4 matrix cores "
                        "with T activation terms (moe_route + moe_expert_fwd_mx_mma per layer "
                        "call) instead of moe_layer_fwd")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 2 GiB device copy (HBM counter calibration)")
    p.add_argument("--calibrate-read", action="store_true",
                   help="only measure the achievable HBM read rate (a plain streaming read "
                        "over 16 GiB, and single launches of one K3 layer's bytes) and print it")
    p.add_argument("--read-windows", default="",
                   help="with --calibrate-read: comma-separated window sizes in MB; one line "
                        "per window with the single-launch rate and time of a plain read of "
                        "that many bytes")
    return p.parse_args()


def calibrate_copy():
    import torch
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copied {n} bytes x 3")


def read_bandwidth(window_bytes: int = 323_018_944, total_gib: int = 16, passes: int = 4):
    """The achievable HBM read rate on this GPU, measured with a plain
    streaming read (synth.device.stream_read: 16-byte non-temporal loads,
    four in flight per thread, grid-stride), the best of 1024, 2048 and 4096
    workgroups of 256 threads:

    * streaming: the whole 16 GiB buffer (64x the 256 MB last-level cache)
      per launch, best of `passes`;
    * single launch: one launch per window of `window_bytes` (by default one
      K3 layer call's algorithmic bytes), consecutive launches reading
      consecutive windows of the 16 GiB buffer so that no window is read
      twice within 50 launches; the average per launch, ramp and tail
      included (the same situation as one layer kernel).
    Returns (streaming GB/s, single-launch GB/s)."""
    import torch
    import synth.device as sd
    n = total_gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w = (window_bytes + 4095) // 4096 * 4096
    nwin = n // w
    nb = window_bytes // 16 * 16
    best, single = 0.0, 0.0
    for blocks in (1024, 2048, 4096):
        sd.stream_read(buf.data_ptr(), n, blocks, sink.data_ptr(), st.cuda_stream)     # warm-up
        for _ in range(passes):
            a.record(st)
            sd.stream_read(buf.data_ptr(), n, blocks, sink.data_ptr(), st.cuda_stream)
            b.record(st)
            torch.cuda.synchronize()
            best = max(best, n / (a.elapsed_time(b) * 1e-3) / 1e9)
        launches = 100
        a.record(st)
        for i in range(launches):
            sd.stream_read(buf.data_ptr() + (i % nwin) * w, nb, blocks, sink.data_ptr(), st.cuda_stream)
        b.record(st)
        torch.cuda.synchronize()
        single = max(single, nb * launches / (a.elapsed_time(b) * 1e-3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return best, single


KERNEL_SRC = tuple(os.path.join(ROOT, "routed_expert_fp4_amd", "csrc", f)
                   for f in ("routed_fp4.hip", "common.h"))
COUNTERS = os.path.join(ROOT, "profiles", "k_moe1_k3_stack_nvfp4_hbm_counters.md")


def measured_traffic():
    """HBM bytes per layer-kernel launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy's reading), or None
    when the kernel source has changed since the counters were taken."""
    import re
    try:
        text = open(COUNTERS).read()
    except OSError:
        return None
    h = re.search(r"code-sha256 [^:]*: ([0-9a-f]{64})", text)
    t = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    if not h or not t:
        return None
    if code_sha256(KERNEL_SRC) != h.group(1):
        return None
    return int(t.group(1))


def code_sha256(paths) -> str:
    """sha256 of C/HIP sources (concatenated in the given order) with comments
    and blank space removed, so an edit to comments alone does not void
    measurements of the same code."""
    import hashlib
    import re
    text = "".join(open(p).read() for p in paths)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = "\n".join(line.strip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(text.encode()).hexdigest()


def check_error_word(ws, what: str):
    """The single-launch decode kernel sets the uint32 at byte 16 of its
    workspace when one of its bounded waits gives up (its outputs are then
    undefined): a timing taken with it set is not a measurement."""
    import torch
    torch.cuda.synchronize()
    if int(ws.tensor[4].item()) != 0:
        log(f"{what}: the decode kernel's error word is set (a bounded wait expired); "
            "no figure is reported")
        sys.exit(3)


def expert_bytes(spec) -> int:
    return spec.expert_bytes()


def cpu_baseline(wl, layers: int, max_tokens: int = 8, threads: int = 0, max_experts: int = 0,
                 keep: dict = None):
    """The oracle as it is, on `layers` layer calls of the workload with at
    most `max_tokens` tokens each (the first tokens of the call); input
    regeneration (the synthetic bank bytes) is excluded from the timing.  Each
    distinct selected expert is dequantised once per call.  threads: the
    oracle's OpenMP threads (0: all it has).  max_experts > 0 times only the
    first max_experts distinct experts of each call and scales their time by
    the call's (token, slot) pairs over the sampled experts' pairs (the
    router, top-k, weights and combine are timed whole).  keep (a dict): with
    every expert computed, receives layer 0's inputs and oracle outputs (x,
    Wr, idx, out) for the parity sample."""
    import numpy as np
    import oracle
    import synth
    oracle.build()
    L_ = oracle.lib()
    prev = int(L_.orc_threads())
    if threads:
        L_.orc_set_threads(threads)
    try:
        total = 0.0
        C = min(wl.C, max_tokens)
        sampled = []
        for l in range(layers):
            spec = wl.bank(l % wl.layers)
            Wr, x = synth.layer_inputs(wl, l % wl.layers, pool=0)
            x = np.ascontiguousarray(x[:C])
            L = oracle.router_logits(x, Wr)
            idx = oracle.topk(L, wl.k)
            uniq = np.unique(idx)
            take = uniq if not max_experts else uniq[:max_experts]
            tensors = {int(e): synth.expert_tensors(spec, int(e)) for e in take}
            t0 = time.perf_counter()
            L = oracle.router_logits(x, Wr)
            idx = oracle.topk(L, wl.k)
            t_route = time.perf_counter() - t0
            ys = np.zeros((C, wl.k, wl.H))
            t1 = time.perf_counter()
            pairs = 0
            for e in take:
                t = tensors[int(e)]
                g = t["globals"]
                Wg = oracle.dequant(spec.fmt, t["gate_codes"], t["gate_scales"], g[0])
                Wu = oracle.dequant(spec.fmt, t["up_codes"], t["up_scales"], g[1])
                Wd = oracle.dequant(spec.fmt, t["down_codes"], t["down_scales"], g[2])
                for tok, slot in zip(*np.nonzero(idx == e)):
                    ys[tok, slot] = oracle.expert_ffn(Wg, Wu, Wd, x[tok])
                    pairs += 1
            t_exp = (time.perf_counter() - t1) * (C * wl.k / pairs)
            t2 = time.perf_counter()
            outs = [oracle.combine(oracle.route_weights(L[tok, idx[tok]]), ys[tok]) for tok in range(C)]
            total += t_route + t_exp + (time.perf_counter() - t2)
            if keep is not None and l == 0 and not max_experts:
                keep.update(x=x, Wr=Wr, idx=idx, out=np.stack(outs))
            sampled.append(len(take))
        cores = int(L_.orc_threads())
    finally:
        L_.orc_set_threads(prev)
    us = total / (layers * C) * 1e6
    sample = f"{layers} layer call(s) of {C} token(s) of the same workload (pool draw 0"
    if C < wl.C:
        sample += f", the first {C} of the call's {wl.C} tokens"
    sample += "): router, top-k, weights, "
    if max_experts:
        sample += (f"dequantisation and FFNs of {sampled[0]} of the call's distinct selected "
                   f"experts, their time scaled by all (token, slot) pairs over theirs, ")
    else:
        sample += "dequantisation of each distinct selected expert, the expert FFNs, "
    sample += "and the combine; bank byte regeneration not timed"
    return {"value": us, "unit": "us/token per MoE layer", "cores": cores,
            "kind": "oracle", "sample": sample}


def parity_sample(rf, bank, ref, wl, ws, dev):
    """The timed path on the oracle's own sample (layer 0, pool draw 0, the
    call's tokens): outputs against the fp64 oracle at the library's bar, and
    the tokens whose selection equals the oracle's (a token that differs is a
    near-tie only if the tests' certified bound allows it; here it is just
    counted)."""
    import numpy as np
    import torch
    import oracle
    C = ref["x"].shape[0]
    x = torch.from_numpy(np.ascontiguousarray(ref["x"])).to(dev)
    Wr = torch.from_numpy(np.ascontiguousarray(ref["Wr"])).to(dev)
    out = torch.empty((C, wl.H), dtype=torch.float32, device=dev)
    idx = torch.empty((C, wl.k), dtype=torch.int32, device=dev)
    rf.moe_layer_fwd(bank, Wr, x, C, wl.k, out, topk_idx_out=idx, ws=ws)
    torch.cuda.synchronize()
    check_error_word(ws, "parity sample")
    got = out.cpu().numpy()
    r, m = oracle.rel_l2(got, ref["out"]), oracle.max_abs_ratio(got, ref["out"])
    same = int(np.sum(np.all(idx.cpu().numpy() == ref["idx"], axis=1)))
    return {"rel_l2": float(f"{r:.3e}"), "max_abs_ratio": float(f"{m:.3e}"),
            "tokens": C, "tokens_with_oracle_selection": same,
            "within_bar": bool(r <= 2e-5 and m <= 1e-4),
            "bar": "rel-L2 <= 2e-5 and max-abs <= 1e-4 x max|ref| (the tests' bar)",
            "sample": "layer 0, pool draw 0, the call's tokens, through moe_layer_fwd, "
                      "against the fp64 CPU oracle"}


def cpu_baseline_latent(wl, keep: dict = None):
    """The oracle as it is on one token of the latent workload's first layer:
    router, routed_down, dequantisation and FFN of each selected routed expert,
    the combine, the norm, routed_up and the shared experts; bank byte
    regeneration (synth) is done before the timing.  keep (a dict) receives
    the token, the oracle's selection and output for the parity sample."""
    import numpy as np
    import oracle
    import synth
    oracle.build()
    Wr, x, Wd, Wu, g = synth.latent_inputs(wl, 0, pool=0, C=1)
    _, idx, _ = oracle.route(x, Wr, wl.k)
    rs, ss = wl.routed_bank(0), wl.shared_bank(0)
    rt = {int(e): synth.expert_tensors(rs, int(e)) for e in np.unique(idx)}
    st = {j: synth.expert_tensors(ss, j) for j in range(wl.n_shared)}

    def deq(spec, t):
        gl = t["globals"]
        return (oracle.dequant(spec.fmt, t["gate_codes"], t["gate_scales"], gl[0]),
                oracle.dequant(spec.fmt, t["up_codes"], t["up_scales"], gl[1]),
                oracle.dequant(spec.fmt, t["down_codes"], t["down_scales"], gl[2]))

    t0 = time.perf_counter()
    rc = {e: deq(rs, t) for e, t in rt.items()}
    sc = {j: deq(ss, t) for j, t in st.items()}
    ref = oracle.latent_layer(wl, Wr, x, Wd, Wu, g, routed_cache=rc, shared_cache=sc)
    us = (time.perf_counter() - t0) * 1e6
    if keep is not None:
        keep.update(x=x, idx=idx, out=ref["out"])
    return {"value": us, "unit": "us/token per latent MoE layer",
            "cores": int(oracle.lib().orc_threads()), "kind": "oracle",
            "sample": "1 token of layer 0 (pool draw 0): dequantisation of the selected routed "
                      "experts and the shared experts, router, routed_down, expert FFNs, combine, "
                      "norm, routed_up, shared FFNs; bank byte regeneration not timed"}


def bench_latent(args, wl):
    """Latent MoE layers (router on x, routed_down, routed experts in the
    latent width, RMS norm of their sum, routed_up, shared experts), one
    moe_latent_layer_fwd call per layer per step."""
    import numpy as np
    import torch
    import routed_expert_fp4_amd as rf
    import synth
    import synth.device as sd

    if args.tokens > 0:
        wl = wl.with_(C=args.tokens)
    C, pool = wl.C, POOL
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    t_setup = time.perf_counter()
    layers, xs, keep = [], [], []
    for l in range(wl.layers):
        rs, ss = wl.routed_bank(l), wl.shared_bank(l)
        rb = rf.Bank(wl.fmt, wl.E, wl.L, wl.I, device=dev)
        sb = rf.Bank(wl.fmt, wl.n_shared, wl.H, wl.I_shared, device=dev)
        sd.fill_bank(rb.storage.data_ptr(), rb.offsets, rb.stride, rs, stream.cuda_stream)
        sd.fill_bank(sb.storage.data_ptr(), sb.offsets, sb.stride, ss, stream.cuda_stream)
        Wr, x, Wd, Wu, g = synth.latent_inputs(wl, l, pool=0, C=pool * C)
        t = [torch.from_numpy(Wr).to(dev), torch.from_numpy(Wd.view(np.int16)).to(dev),
             torch.from_numpy(g).to(dev), torch.from_numpy(Wu.view(np.int16)).to(dev)]
        layers.append(rf.LatentLayer(t[0], t[1], t[2], wl.eps, t[3], rb, sb))
        xs.append(torch.from_numpy(x).to(dev))
        keep.append((rb, sb, t))
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f}s: {wl.layers} latent layers")
    ws = rf.LatentWorkspace(layers[0], wl.k, C, device=dev)
    outs = [torch.empty((C, wl.H), dtype=torch.float32, device=dev) for _ in range(wl.layers)]
    idx = [[torch.empty((C, wl.k), dtype=torch.int32, device=dev) for _ in range(pool)]
           for _ in range(wl.layers)]

    def step(i):
        j = i % pool
        for l in range(wl.layers):
            rf.moe_latent_layer_fwd(layers[l], xs[l][j * C:(j + 1) * C], C, wl.k, outs[l],
                                    idx[l][j], None, ws)

    for i in range(max(args.warmup, pool)):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    check_error_word(ws, "latent layer timing")
    ms_step = e0.elapsed_time(e1) / args.steps
    us_call = ms_step * 1000.0 / wl.layers
    uniq = np.mean([len(np.unique(idx[l][j].cpu().numpy())) for l in range(wl.layers)
                    for j in range(pool)])
    rexp, sexp = wl.routed_bank(0).expert_bytes(), wl.shared_bank(0).expert_bytes()
    dense_bytes = wl.E * wl.H * 4 + 2 * wl.L * wl.H * 2 + wl.L * 4
    alg_bytes = uniq * rexp + wl.n_shared * sexp + dense_bytes + 2 * C * wl.H * 4
    gbps = alg_bytes / (us_call * 1e-6) / 1e9
    fmt = "nvfp4" if wl.fmt == synth.FMT_NV else "mxfp4"
    if C == 1:
        kernels = ("k_lat_in (routed_down + the shared experts' gate/up, with the shared "
                   "selection), k_moe1 (router on the hidden state + routed experts, one launch), "
                   "k_lat_out (the shared experts' down + norm + routed_up)")
    else:
        kernels = ("k_gemv (routed_down, with the shared selection and dispatch table), "
                   "k_route + k_btopk (router and routed dispatch table), routed experts and "
                   "then shared experts (k_dstream<GU> + k_dstream<DN> + k_bcombine each), "
                   "k_gemv (norm + routed_up)")
    result = {
        "metric": "latent MoE layer decode µs/token + achieved HBM GB/s (% of peak)",
        "value": round(us_call / C, 3),
        "unit": "us/token per latent MoE layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": f"synthetic (seeded {fmt} banks generated on device, bf16 N(0,1/K) dense "
                "matrices, fp32 N(0,1) tokens, N(0,0.02) router)",
        "config": {"workload": f"{wl.name}: {wl.layers} latent MoE layer(s): router on H {wl.H}, "
                               f"routed_down {wl.H}->{wl.L}, {wl.E} routed experts top-{wl.k} "
                               f"(H {wl.L}, I {wl.I}), norm, routed_up {wl.L}->{wl.H}, "
                               f"{wl.n_shared} shared experts (H {wl.H}, I {wl.I_shared}), {fmt}, "
                               f"{C} token(s) per call",
                   "layers": wl.layers, "experts": wl.E, "top_k": wl.k, "hidden": wl.H,
                   "latent": wl.L, "inter": wl.I, "shared": wl.n_shared, "format": fmt,
                   "tokens_per_call": C},
        "us_per_call": round(us_call, 3),
        "tokens_per_s": round(1000.0 * C / ms_step, 2),
        "distinct_experts_per_call": round(float(uniq), 2),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": kernels + " per moe_latent_layer_fwd call",
                     "bytes_per_launch": int(alg_bytes), "us_per_launch": round(us_call, 3)},
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        ref = {}
        result["cpu_baseline"] = cpu_baseline_latent(wl, keep=ref)
        if ref and C == ref["x"].shape[0]:
            import oracle
            xg = torch.from_numpy(np.ascontiguousarray(ref["x"])).to(dev)
            og = torch.empty((C, wl.H), dtype=torch.float32, device=dev)
            ig = torch.empty((C, wl.k), dtype=torch.int32, device=dev)
            rf.moe_latent_layer_fwd(layers[0], xg, C, wl.k, og, ig, None, ws)
            torch.cuda.synchronize()
            check_error_word(ws, "parity sample")
            got = og.cpu().numpy()
            r, m = oracle.rel_l2(got, ref["out"]), oracle.max_abs_ratio(got, ref["out"])
            result["parity_sample"] = {
                "rel_l2": float(f"{r:.3e}"), "max_abs_ratio": float(f"{m:.3e}"), "tokens": C,
                "tokens_with_oracle_selection": int(np.sum(np.all(ig.cpu().numpy() == ref["idx"], axis=1))),
                "within_bar": bool(r <= 2e-5 and m <= 1e-4),
                "bar": "rel-L2 <= 2e-5 and max-abs <= 1e-4 x max|ref| (the tests' bar)",
                "sample": "layer 0, pool draw 0, one token, through moe_latent_layer_fwd, "
                          "against the fp64 CPU oracle"}
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.calibrate_read:
        import synth.device as sd
        if not os.path.exists(sd.LIB):
            sd.build()
        torch.cuda.set_device(0)
        if args.read_windows:
            for mb in (float(v) for v in args.read_windows.split(",")):
                nbytes = int(mb * 1e6)
                streaming, single = read_bandwidth(nbytes, passes=2)
                print(json.dumps({"calibration": "HBM read rate, plain streaming read (16-byte "
                                                 "non-temporal loads)",
                                  "window_mb": mb, "single_launch_gbps": round(single, 1),
                                  "single_launch_us": round(nbytes / (single * 1e3), 2),
                                  "streaming_16GiB_gbps": round(streaming, 1),
                                  "peak_gbps": HBM_PEAK_GBPS}), flush=True)
            return
        streaming, single = read_bandwidth()
        print(json.dumps({"calibration": "HBM read rate, plain streaming read (16-byte "
                                         "non-temporal loads)",
                          "streaming_16GiB_gbps": round(streaming, 1),
                          "single_launch_323MB_gbps": round(single, 1),
                          "peak_gbps": HBM_PEAK_GBPS}), flush=True)
        return

    import routed_expert_fp4_amd as rf
    if not os.path.exists(rf.LIB_PATH):
        from routed_expert_fp4_amd import build
        build.build_library()
    import synth
    import synth.device as sd
    if not os.path.exists(sd.LIB):
        sd.build()

    if args.workload in synth.LATENT_WORKLOADS:
        torch.cuda.set_device(0)
        bench_latent(args, synth.LATENT_WORKLOADS[args.workload])
        return
    wl = synth.WORKLOADS[args.workload]
    if args.tokens > 0:
        wl = wl.with_(C=args.tokens)
    pool = POOL if wl.C <= 16 else 2
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    t_setup = time.perf_counter()

    # ---- resident bank: every layer's experts in HBM ----
    banks, wrs, xs = [], [], []
    for l in range(wl.layers):
        spec = wl.bank(l)
        b = rf.Bank(wl.fmt, wl.E, wl.H, wl.I, device=dev)
        sd.fill_bank(b.storage.data_ptr(), b.offsets, b.stride, spec, stream.cuda_stream)
        banks.append(b)
        Wr, x = synth.layer_inputs(wl, l, pool=0, C=pool * wl.C)
        wrs.append(torch.from_numpy(Wr).to(dev))
        xs.append(torch.from_numpy(x).to(dev))
    torch.cuda.synchronize()
    resident = sum(b.storage.numel() for b in banks)
    need = wl.layers * wl.E * banks[0].stride
    if resident < need:
        raise SystemExit("bank not fully resident")
    log(f"setup {time.perf_counter() - t_setup:.1f}s: {wl.layers} layers, "
        f"{resident / 1e9:.1f} GB resident bank")

    C = wl.C
    ws = rf.Workspace(wl.E, wl.H, wl.I, wl.k, C, device=dev)
    outs = [torch.empty((C, wl.H), dtype=torch.float32, device=dev) for _ in range(wl.layers)]

    def step(i):
        j = i % pool
        for l in range(wl.layers):
            rf.moe_layer_fwd(banks[l], wrs[l], xs[l][j * C:(j + 1) * C], C, wl.k, outs[l], ws=ws)

    if args.mx_mma:
        if wl.fmt != synth.FMT_MX:
            raise SystemExit("--mx-mma needs an MXFP4 workload")
        mws = rf.MxMmaWorkspace(banks[0], wl.k, C, args.mx_mma, device=dev)
        ridx = torch.empty((C, wl.k), dtype=torch.int32, device=dev)
        rw = torch.empty((C, wl.k), dtype=torch.float32, device=dev)

        def step(i):  # noqa: F811  (the same step with the experts on the FP4 matrix cores)
            j = i % pool
            for l in range(wl.layers):
                xj = xs[l][j * C:(j + 1) * C]
                rf.moe_route(xj, wrs[l], None, C, wl.H, wl.E, wl.k, ridx, rw, ws)
                rf.moe_expert_fwd_mx_mma(banks[l], xj, C, wl.k, ridx, rw, outs[l], args.mx_mma, mws)

    # ---- whole path ----
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    check_error_word(ws, "layer timing")
    ms_step = e0.elapsed_time(e1) / args.steps
    # one layer call alone, the stream idle before it (events around the call)
    singles = []
    if not args.mx_mma:
        for r in range(7):
            j = r % pool
            torch.cuda.synchronize()
            a1, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a1.record(stream)
            rf.moe_layer_fwd(banks[0], wrs[0], xs[0][j * C:(j + 1) * C], C, wl.k, outs[0], ws=ws)
            b1.record(stream)
            torch.cuda.synchronize()
            singles.append(a1.elapsed_time(b1) * 1000.0)
        check_error_word(ws, "single-call timing")
    us_call = ms_step * 1000.0 / wl.layers          # one moe_layer_fwd call (C tokens)
    us_layer = us_call / C                          # per token per MoE layer

    # ---- the expert work alone (selection given) and the routing alone ----
    idx = [[torch.empty((C, wl.k), dtype=torch.int32, device=dev) for _ in range(pool)]
           for _ in range(wl.layers)]
    wts = [[torch.empty((C, wl.k), dtype=torch.float32, device=dev) for _ in range(pool)]
           for _ in range(wl.layers)]
    for l in range(wl.layers):
        for j in range(pool):
            rf.moe_route(xs[l][j * C:(j + 1) * C], wrs[l], None, C, wl.H, wl.E, wl.k,
                         idx[l][j], wts[l][j], ws)
    torch.cuda.synchronize()

    def expert_step(i):
        j = i % pool
        for l in range(wl.layers):
            rf.moe_expert_fwd(banks[l], xs[l][j * C:(j + 1) * C], C, wl.k, idx[l][j], wts[l][j],
                              outs[l], ws)

    def route_step(i):
        j = i % pool
        for l in range(wl.layers):
            rf.moe_route(xs[l][j * C:(j + 1) * C], wrs[l], None, C, wl.H, wl.E, wl.k,
                         idx[l][j], wts[l][j], ws)

    def timed(fn, n):
        for i in range(max(2, args.warmup // 2)):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (n * wl.layers) * 1000.0     # us per layer call

    us_expert = timed(expert_step, args.steps) if not args.layer_only else float("nan")
    us_route = timed(route_step, args.steps) if not args.layer_only else float("nan")
    check_error_word(ws, "expert-only timing")
    # distinct experts per call
    uniq = np.mean([len(np.unique(idx[l][j].cpu().numpy())) for l in range(wl.layers)
                    for j in range(pool)])
    spec0 = wl.bank(0)
    sel_bytes = uniq * expert_bytes(spec0)
    router_bytes = wl.E * wl.H * 4
    gbps_layer = sel_bytes / (us_call * 1e-6) / 1e9
    # the layer kernel's algorithmic bytes: router weights + selected experts
    # (+ x in, y out, negligible but counted)
    alg_bytes = router_bytes + sel_bytes + 2 * C * wl.H * 4
    gbps_kernel = alg_bytes / (us_call * 1e-6) / 1e9
    fmt = "nvfp4" if wl.fmt == synth.FMT_NV else "mxfp4"
    if args.mx_mma:
        kernel = (f"k_brouter + k_btopk, then k_mq_split + k_mcount/k_mscan/k_mscatter + "
                  f"k_mgemm<GU> + k_mq_split + k_mgemm<DN> + k_mcombine ({args.mx_mma} e4m3 "
                  "activation terms) per layer call")
    elif C == 1 and wl.name != "tiny":
        kernel = "k_moe1 (whole layer, one launch per moe_layer_fwd call)"
    elif wl.name == "tiny":
        kernel = "k_route + k_btopk + k_gate_up + k_down (+ k_zero_uncovered) per moe_layer_fwd call"
    elif C <= 16:
        kernel = "k_route + k_btopk + k_dstream<GU> + k_dstream<DN> + k_bcombine per moe_layer_fwd call"
    else:
        kernel = ("k_brouter + k_btopk + k_bsplit/k_bcount/k_bscan/k_bscatter + k_bdma or k_bmm "
                  "(gate/up, down) + k_bcombine per moe_layer_fwd call")

    result = {
        "metric": METRIC,
        "value": round(us_layer, 3),
        "unit": "us/token per MoE layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": f"synthetic (seeded {fmt} bank generated on device, fp32 N(0,1) tokens, "
                "N(0,0.02) router)",
        "config": {"workload": f"{wl.name}: {wl.layers} MoE layer(s) x {wl.E} experts, top-{wl.k}, "
                               f"H {wl.H}, I {wl.I}, {fmt}, {C} token(s) per call, "
                               + ("uniform (natural) routing" if wl.routing == "natural"
                                  else f"Zipf s={wl.zipf_s} routing"),
                   "layers": wl.layers, "experts": wl.E, "top_k": wl.k, "hidden": wl.H,
                   "inter": wl.I, "format": fmt, "tokens_per_call": C},
        "us_per_call": round(us_call, 3),
        "us_single_call": round(float(np.median(singles)), 3) if singles else None,
        "hbm_gbps_selected_expert_bytes": round(gbps_layer, 1),
        "hbm_frac_of_peak": round(gbps_layer / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(1000.0 * C / ms_step, 2),
        "distinct_experts_per_call": round(float(uniq), 2),
        "selected_expert_bytes_per_call": int(sel_bytes),
        "router_bytes_per_layer": router_bytes,
        "us_per_call_route": None if args.layer_only else round(us_route, 3),
        "us_per_call_experts": None if args.layer_only else round(us_expert, 3),
        "roofline": {"bound": "hbm", "achieved": round(gbps_kernel, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps_kernel / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic() if wl.name == "k3_stack" else None,
                     "kernel": kernel,
                     "bytes_per_launch": int(alg_bytes),
                     "us_per_launch": round(us_call, 3)},
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_read_calibration:
        streaming, single = read_bandwidth(window_bytes=max(16, int(alg_bytes) // 16 * 16))
        result["roofline"]["achievable_read_gbps"] = {
            "streaming_16GiB": round(streaming, 1),
            "single_launch_same_bytes": round(single, 1),
            "how": "plain streaming read (bench.py --calibrate-read), one launch per window of "
                   "the layer kernel's algorithmic bytes"}
        result["roofline"]["frac_of_single_launch_read"] = round(gbps_kernel / single, 4)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        ref = {}
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_layers, keep=ref)
        if ref and ref["x"].shape[0] == C and not args.mx_mma:
            result["parity_sample"] = parity_sample(rf, banks[0], ref, wl, ws, dev)
        log("timing the CPU oracle on one core (sampled experts) ...")
        result["cpu_baseline_1core"] = cpu_baseline(wl, 1, threads=1,
                                                    max_experts=2 if wl.C == 1 else 4)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
