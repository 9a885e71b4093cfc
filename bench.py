"""Benchmark: NVFP4 MoE decode layer calls/s and achieved HBM bandwidth, batch 1.

One step = one call of the whole decode hot path (router, top-k, gate|up GEMV
with in-register dequant and clamped SwiGLU, down GEMV, weighted combine and
shared expert) on one token, through the C ABI (ft_moe_nvfp4_decode).

Inputs are synthetic and already resident in HBM when timing starts.  Calls
cycle over L distinct layer instances (different weights and activations) so
that the bytes touched per cycle exceed 4x the 256 MB Infinity Cache: the
measured bandwidth is HBM bandwidth, not cache bandwidth.

Prints one JSON line (rank 0, N = 1).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E peak, 8 TB/s
MALL_BYTES = 256 << 20      # Infinity Cache
METRIC = "NVFP4 MoE decode: layer calls/s + achieved HBM GB/s (% of peak), batch 1"


def algorithmic_bytes(w, ids: np.ndarray) -> int:
    """Bytes a call must move at least once: the router weights, the activations
    in and out, and the codes, scales and global scales of every distinct
    selected expert (plus the shared expert and its gate vector)."""
    H, I = w.hidden, w.inter

    def expert_bytes(inter):
        if getattr(w, "codec", "nvfp4") == "fp8":   # e4m3 codes + fp32 scale per 128x128 block
            return 3 * inter * H + 4 * ((2 * inter // 128) * (H // 128) + (H // 128) * (inter // 128))
        return (2 * inter * H) // 2 + (2 * inter * H) // 16 + (H * inter) // 2 + (H * inter) // 16 + 12

    per_expert = expert_bytes(I)
    b = w.num_experts * H * 4                  # router weights, fp32
    if w.hot_experts > 0:
        b += w.num_experts * 4                 # router bias
    T = ids.shape[0]
    b += 2 * T * H * 2                         # x in, y out (bf16)
    b += len(np.unique(ids)) * per_expert
    if w.shared_inter > 0:
        b += expert_bytes(w.shared_inter)
        b += H * 2                             # shared gate vector
    return b


ROOT = os.path.dirname(os.path.abspath(__file__))
DECODE_KERNEL = "moe_decode_fused_kernel"
DECODE_SOURCES = ("nvfp4_mixture_experts_amd/csrc/decode_fused.hip",
                  "nvfp4_mixture_experts_amd/csrc/ftmoe_device.hpp",
                  "nvfp4_mixture_experts_amd/csrc/ftmoe_kernels.hpp",
                  "nvfp4_mixture_experts_amd/csrc/handoff.hpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch of the decode kernel from the committed rocprofv3 --pmc
    summary (FETCH_SIZE and WRITE_SIZE runs, scaled by a plain copy of known size),
    or None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{DECODE_KERNEL}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                kv[k.strip()] = v.strip().strip("`")
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    try:
        fetch = float(kv["fetch_bytes_per_launch"])
        write = float(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None
    return {"bytes": fetch + write, "fetch": fetch, "write": write}


def _time_oracle(layer, x, tokens: int, seconds: float, openmp: bool):
    import oracle
    oracle.moe_layer(layer, x[:1], openmp=openmp)        # warm-up (and library load)
    n = 0
    t0 = time.perf_counter()
    while True:
        i = (n * tokens) % x.shape[0]
        oracle.moe_layer(layer, x[i:i + tokens], openmp=openmp)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return n, el


def cpu_baseline(w, seconds: float = 12.0) -> dict:
    """The CPU oracle, as it stands, on a bounded sample of the same workload: its
    OpenMP build (independent rows spread over every host core; same bits as the
    plain build) and, for reference, the plain single-threaded build."""
    import oracle
    from nvfp4_mixture_experts_amd import synth
    layer = synth.make_layer(w)
    x = synth.make_tokens(w, tokens=64, stream="cpu_baseline")
    cores = oracle.threads(openmp=True)
    n, el = _time_oracle(layer, x, w.tokens, seconds / 2, openmp=True)
    n1, el1 = _time_oracle(layer, x, w.tokens, seconds / 2, openmp=False)
    return {"value": n / el, "unit": "calls/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} calls of {w.name} ({w.tokens} token(s) each) on instance 0 in "
                      f"{el:.1f} s, C oracle (fp64) built with OpenMP on {cores} threads; "
                      f"host {platform.processor() or 'cpu'}, nproc {os.cpu_count()}",
            "single_thread_value": n1 / el1,
            "single_thread_sample": f"{n1} calls in {el1:.1f} s, plain single-threaded build"}


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def prefill_flops(w, T: int) -> float:
    """Useful expert FLOP of one prefill chunk: every routed (token, slot) pair and
    every token of the shared expert runs gate|up (2I x H) and down (H x I)."""
    per_routed = 2.0 * (2 * w.inter * w.hidden + w.hidden * w.inter)
    per_shared = 2.0 * (2 * w.shared_inter * w.hidden + w.hidden * w.shared_inter)
    return T * w.top_k * per_routed + T * per_shared


def cpu_baseline_prefill(w, seconds: float) -> dict:
    import oracle
    from nvfp4_mixture_experts_amd import synth
    layer = synth.make_layer(w)
    x = synth.make_tokens(w, tokens=64, stream="cpu_baseline")
    cores = oracle.threads(openmp=True)
    n, el = _time_oracle(layer, x, 1, seconds / 2, openmp=True)
    n1, el1 = _time_oracle(layer, x, 1, seconds / 2, openmp=False)
    return {"value": n / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} tokens of {w.name} (routing, experts, shared expert) one at a time "
                      f"on instance 0 in {el:.1f} s, C oracle (fp64) built with OpenMP on "
                      f"{cores} threads; nproc {os.cpu_count()}",
            "single_thread_value": n1 / el1,
            "single_thread_sample": f"{n1} tokens in {el1:.1f} s, plain single-threaded build"}


def measure_prefill(args, w, steps: int, warmup: int) -> dict:
    """A prefill chunk: ft_moe_route then ft_moe_nvfp4_prefill over w.tokens tokens,
    cycling over 2 layer instances (each touches ~1 GB); MFMA utilisation of the useful
    expert FLOP against the dense bf16 peak, whole call (router included)."""
    import torch
    from nvfp4_mixture_experts_amd import device, ftmoe, synth
    dev = torch.device("cuda:0")
    T = w.tokens
    L = 2
    layers, xs = [], []
    for l in range(L):
        d = synth.make_layer_device(w, l, dev)
        layers.append(device.upload_canonical(w, d["w_router"], d["bias"], d["routed"], d["shared"],
                                              d["shared_gate"], dev))
        del d
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed + 7919 * l + 1)
        xs.append(torch.randn((T, w.hidden), generator=g, device=dev).to(torch.bfloat16))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    desc = layers[0].desc
    wsr = ftmoe.alloc_workspace(desc, T, ftmoe.PATH_ROUTE, dev)
    wsp = ftmoe.alloc_workspace(desc, T, ftmoe.PATH_PREFILL, dev)
    y = torch.empty((T, w.hidden), dtype=torch.bfloat16, device=dev)
    ids = torch.empty((T, w.top_k), dtype=torch.int32, device=dev)
    wt = torch.empty((T, w.top_k), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def call(i):
        dl = layers[i % L]
        ftmoe.ft_moe_route(desc, xs[i % L], dl.w_router, dl.bias, ids, wt, wsr, stream=stream)
        ftmoe.ft_moe_nvfp4_prefill(desc, xs[i % L], ids, wt, dl.routed, dl.shared, dl.shared_gate,
                                   y, wsp, stream=stream)

    warm = max(min(warmup, 8), L)
    for i in range(warm):
        call(i)
    torch.cuda.synchronize()
    steps = max(L, min(steps, 40))
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        call(i)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    flops = prefill_flops(w, T)
    tflops = flops / (ms * 1e-3) / 1e12
    del layers, xs
    torch.cuda.empty_cache()
    return {
        "workload": w.name, "entry": "ft_moe_route + ft_moe_nvfp4_prefill",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "steps": steps, "warmup": warm,
        "ms_per_step": round(ms, 4),
        "config": {"workload": w.name, "experts": w.num_experts, "hidden": w.hidden,
                   "inter": w.inter, "top_k": w.top_k, "tokens": T,
                   "shared_inter": w.shared_inter, "layer_instances": L},
        "roofline": {"kernel": "route + grouped GEMMs (whole call)", "bound": "mfma",
                     "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "useful_flop_per_call": flops},
        "launch": "eager, one route and one prefill call per step",
    }


def run_prefill(args, w) -> int:
    m = measure_prefill(args, w, args.steps, args.warmup)
    out = {"metric": "NVFP4 MoE prefill chunk: tokens/s + MFMA utilisation of useful expert FLOP",
           "value": m["value"], "unit": "tokens/s", "n_gpus": 1, "steps": m["steps"],
           "warmup": m["warmup"], "ms_per_step": m["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": m["config"], "roofline": m["roofline"], "launch": m["launch"]}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_prefill(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA


def _graph_reps(torch, calls_per_graph, make_call, reps: int):
    """Capture `reps` graphs of `calls_per_graph` calls (make_call(i, stream) enqueues
    call i), replay each once, return the per-call ms of each replay."""
    stream = torch.cuda.current_stream()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    graphs = []
    for r in range(reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(calls_per_graph):
                    make_call(r * calls_per_graph + i, cap)
        graphs.append(g)
    torch.cuda.synchronize()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    out = []
    for g in graphs:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / calls_per_graph)
    return out


def measure_linear(args, lw, steps: int, reps: int) -> dict:
    """The per-tensor FP8 W8A8 q|k|v projection (ft_fp8_linear, row-wise form): weights
    cycled over enough instances to defeat the Infinity Cache when the call is
    weight-bound; roofline HBM for up to 64 tokens, fp8 MFMA above."""
    import torch
    from nvfp4_mixture_experts_amd import ftmoe, synth
    dev = torch.device("cuda:0")
    M, K, N = lw.tokens, lw.hidden, lw.out_rows
    wbytes = N * K
    L = max(1, math.ceil(4 * MALL_BYTES / wbytes)) if M <= 64 else 1
    g = torch.Generator(device=dev)
    g.manual_seed(lw.seed)
    table = torch.tensor(synth.FP8_FINITE_BYTES, dtype=torch.uint8, device=dev)
    ws_ = [table[torch.randint(0, 254, (N, K), generator=g, device=dev)] for _ in range(L)]
    rows = torch.from_numpy(synth.make_fp8_linear(lw).row_scales()).to(dev)
    x = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    wsp = ftmoe.fp8_linear_workspace(M, K, dev)

    def call(i, s):
        ftmoe.ft_fp8_linear(x, ws_[i % L], rows, y, wsp, stream=s)

    for i in range(max(L, 4)):
        call(i, torch.cuda.current_stream())
    torch.cuda.synchronize()
    n = max(steps, L) if M <= 64 else max(2, min(steps, 40))
    per = _graph_reps(torch, n, call, reps)
    ms = float(np.median(per))
    flops = 2.0 * M * N * K
    if M <= 64:
        b = wbytes + 2 * M * K + 2 * M * N + 4 * N
        achieved = b / (ms * 1e-3) / 1e9
        one = M <= 8 and M * K <= 16384 and K <= 2048  # the library's one-launch form
        roof = {"kernel": ("fp8 linear call (quantise + GEMV in one launch)" if one
                           else "fp8 linear call (amax, quantise, GEMM)"), "bound": "hbm",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                "algorithmic_bytes_per_launch": b}
    else:
        tf = flops / (ms * 1e-3) / 1e12
        roof = {"kernel": "fp8 linear call (amax, quantise, GEMM)", "bound": "mfma",
                "achieved": round(tf, 1), "peak": FP8_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / FP8_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                "useful_flop_per_call": flops}
    del ws_
    torch.cuda.empty_cache()
    return {"workload": lw.name, "entry": "ft_fp8_linear", "value": round(1000.0 / ms, 1),
            "unit": "calls/s", "steps": n, "reps": reps, "ms_per_step": round(ms, 6),
            "ms_per_step_reps": [round(v, 6) for v in per],
            "config": {"workload": lw.name, "tokens": M, "hidden": K, "parts": list(lw.parts),
                       "weight_instances": L},
            "roofline": roof, "launch": f"{reps} HIP graphs of {n} calls, median"}


def measure_attn(args, steps: int, reps: int, fmt: int = 2) -> dict:
    """Extend attention (ft_attn_extend): 512 new tokens over a 4096-position NVFP4 cache,
    32 query heads, 4 kv heads, head dim 128, no window.  FLOP = 4 * Hq * d * visible keys
    per query (QK and PV); reported against the bf16 MFMA peak."""
    import torch
    from nvfp4_mixture_experts_amd import ftmoe
    dev = torch.device("cuda:0")
    n_new, P, Hq, Hkv, d = 512, 4096, 32, 4, 128
    g = torch.Generator(device=dev)
    g.manual_seed(3100 + fmt)
    q = torch.randn((n_new, Hq, d), generator=g, device=dev).to(torch.bfloat16)
    kn = torch.randn((n_new, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((n_new, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    kc = torch.randint(0, 256, (P, Hkv, d // 2), generator=g, device=dev, dtype=torch.uint8)
    vc = torch.randint(0, 256, (P, Hkv, d // 2), generator=g, device=dev, dtype=torch.uint8)
    kb = torch.full((P, Hkv, d // 16), 0x30, dtype=torch.uint8, device=dev)
    vb = torch.full((P, Hkv, d // 16), 0x30, dtype=torch.uint8, device=dev)
    out = torch.empty((n_new, Hq, d), dtype=torch.bfloat16, device=dev)

    def call(i, s):
        ftmoe.ft_attn_extend(q, kn, vn, fmt, P, kc, vc, out, 0, kb, vb, 0.25, 0.25, stream=s)

    for i in range(3):
        call(i, torch.cuda.current_stream())
    torch.cuda.synchronize()
    n = max(2, min(steps, 20))
    per = _graph_reps(torch, n, call, reps)
    ms = float(np.median(per))
    keys = sum(P + t + 1 for t in range(n_new))
    flops = 4.0 * Hq * d * keys
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": "attn_extend_nvfp4_p4096_n512", "entry": "ft_attn_extend",
            "value": round(1000.0 / ms, 1), "unit": "calls/s", "steps": n, "reps": reps,
            "ms_per_step": round(ms, 6),
            "config": {"workload": "attn_extend_nvfp4_p4096_n512", "new_tokens": n_new,
                       "prefix": P, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                       "cache_format": "nvfp4", "window": 0},
            "roofline": {"kernel": "attn_extend_kernel", "bound": "mfma",
                         "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 5),
                         "traffic": None, "useful_flop_per_call": flops},
            "launch": f"{reps} HIP graphs of {n} calls, median"}


def stream_read_probe(dev) -> dict:
    """Achievable HBM read bandwidth for context: torch's sum over 4 GiB of fp32 (a
    read-bound library reduction), best of 5."""
    import torch
    n = 1 << 30
    t = torch.ones(n, dtype=torch.float32, device=dev)
    out = torch.empty((), dtype=torch.float32, device=dev)
    torch.sum(t, dim=0, out=out)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(5):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        torch.sum(t, dim=0, out=out)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    del t
    torch.cuda.empty_cache()
    return {"op": "torch.sum over 4 GiB fp32, best of 5", "gbps": round(4 * 2 ** 30 / (best * 1e-3) / 1e9, 1)}


def measure_decode(args, w, steps: int, warmup: int, reps: int, variant: str = "plain") -> dict:
    """Decode calls of workload ``w`` cycling over L layer instances (enough that the
    bytes touched per cycle exceed 4x the Infinity Cache).  Each repetition is one HIP
    graph of exactly ``steps`` calls, continuing the cycle; the median repetition is
    reported.  Inputs are resident in HBM before timing starts.  ``variant`` "slots"
    runs ft_moe_nvfp4_decode_slots over the same bank with a random expert -> slot
    permutation (every expert resident); block-fp8 workloads run ft_moe_fp8_decode."""
    import torch
    from nvfp4_mixture_experts_amd import device, ftmoe, synth
    dev = torch.device("cuda:0")
    fp8 = w.codec == "fp8"
    per_call_guess = algorithmic_bytes(w, np.zeros((w.tokens, w.top_k)) + np.arange(w.top_k))
    L = args.instances or max(2, math.ceil(4 * MALL_BYTES / per_call_guess))
    layers, xs, slot_maps = [], [], []
    for l in range(L):
        if fp8:
            d = synth.make_fp8_layer_device(w, l, dev)
            dl = device.upload_fp8_canonical(w, d["w_router"], d["bias"], d["routed"], d["shared"],
                                             d["shared_gate"], dev)
        else:
            d = synth.make_layer_device(w, l, dev)
            dl = device.upload_canonical(w, d["w_router"], d["bias"], d["routed"], d["shared"],
                                         d["shared_gate"], dev)
        del d
        layers.append(dl)
        if variant == "slots":
            g = torch.Generator(device=dev)
            g.manual_seed(w.seed + 7919 * l + 2)
            slot_maps.append(torch.randperm(w.num_experts, generator=g, device=dev).to(torch.int32))
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed + 7919 * l + 1)
        xs.append(torch.randn((w.tokens, w.hidden), generator=g, device=dev).to(torch.bfloat16))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    desc = layers[0].desc
    ws = ftmoe.alloc_workspace(desc, w.tokens, ftmoe.PATH_DECODE, dev)
    y = torch.empty((w.tokens, w.hidden), dtype=torch.bfloat16, device=dev)
    ids_all = torch.empty((L, w.tokens, w.top_k), dtype=torch.int32, device=dev)
    wts = torch.empty((w.tokens, w.top_k), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def call(i, s):
        dl = layers[i % L]
        if fp8:
            ftmoe.ft_moe_fp8_decode(desc, xs[i % L], dl.w_router, dl.bias, dl.routed, dl.shared,
                                    dl.shared_gate, y, ws, ids_all[i % L], wts, stream=s)
        elif variant == "slots":
            ftmoe.ft_moe_nvfp4_decode_slots(desc, xs[i % L], dl.w_router, dl.bias, dl.routed,
                                            slot_maps[i % L], dl.shared, dl.shared_gate, y, ws,
                                            ids_all[i % L], wts, stream=s)
        else:
            ftmoe.ft_moe_nvfp4_decode(desc, xs[i % L], dl.w_router, dl.bias, dl.routed, dl.shared,
                                      dl.shared_gate, y, ws, ids_all[i % L], wts, stream=s)

    for i in range(max(warmup, L)):
        call(i, stream)
    torch.cuda.synchronize()

    # eager launches (one host call per step), for reference
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    n_eager = min(steps, 20 * L)
    start.record(stream)
    for i in range(n_eager):
        call(i, stream)
    end.record(stream)
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / n_eager

    # timed region: repetition r replays a graph of exactly `steps` calls on
    # instances (r * steps + i) mod L (a decode loop captured once and replayed)
    graphs = []
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    for r in range(reps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                for i in range(steps):
                    call(r * steps + i, cap)
        graphs.append(g)
    torch.cuda.synchronize()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    rep_ms = []
    t0 = time.perf_counter()
    for g in graphs:
        torch.cuda.synchronize()
        start.record(stream)
        g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        rep_ms.append(start.elapsed_time(end) / steps)
    wall = time.perf_counter() - t0
    # secondary, not an HBM figure: every call on layer instance 0, whose weights then
    # stay in the Infinity Cache (untimed by the headline; reported beside it)
    warm_ms = (None if args.no_mall_warm else
               float(np.median(_graph_reps(torch, min(steps, 200), lambda i, s: call(0, s), 3))))
    status = ftmoe.device_status(ws)
    if status != 0:
        raise RuntimeError(f"a device-side wait gave up during timing (status {status:#x})")
    ms_per_step = float(np.median(rep_ms))
    calls_per_s = 1000.0 / ms_per_step

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 18
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ids_np = ids_all.cpu().numpy()
    bytes_per_call = float(np.mean([algorithmic_bytes(w, ids_np[l]) for l in range(L)]))
    gbps = bytes_per_call / (ms_per_step * 1e-3) / 1e9
    grouped = w.tokens >= ftmoe.GROUPED_DECODE_MIN_TOKENS
    traffic = None if (grouped or variant != "plain") else measured_traffic(w.name)
    kernel = ("grouped decode path: route, grouping, gate|up, down, combine (whole call)"
              if grouped else DECODE_KERNEL)
    del graphs, layers, xs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    name = w.name + ("_slots" if variant == "slots" else "")
    return {
        "workload": name,
        "entry": {"plain": "ft_moe_fp8_decode" if fp8 else "ft_moe_nvfp4_decode",
                  "slots": "ft_moe_nvfp4_decode_slots"}[variant],
        "value": round(calls_per_s, 1),
        "unit": "calls/s",
        "steps": steps,
        "reps": reps,
        "ms_per_step": round(ms_per_step, 6),
        "ms_per_step_reps": [round(v, 6) for v in rep_ms],
        "config": {"workload": name, "experts": w.num_experts, "hidden": w.hidden,
                   "inter": w.inter, "top_k": w.top_k, "tokens": w.tokens,
                   "shared_inter": w.shared_inter, "codec": w.codec, "layer_instances": L,
                   "bytes_touched_per_cycle": int(bytes_per_call * L)},
        "achieved_gbps": round(gbps, 1),
        "hbm_peak_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "roofline": {"kernel": kernel, "bound": "hbm",
                     "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else int(round(traffic["bytes"])),
                     "traffic_fetch": None if traffic is None else int(round(traffic["fetch"])),
                     "traffic_write": None if traffic is None else int(round(traffic["write"])),
                     "algorithmic_bytes_per_launch": int(round(bytes_per_call))},
        "wall_s_timed": round(wall, 3),
        "launch": f"{reps} HIP graphs of {steps} calls each (one call per layer instance in "
                  "turn), each replayed once and timed; median reported",
        "eager_ms_per_step": round(eager_ms, 6),
        "mall_warm_l1_ms_per_step": None if warm_ms is None else round(warm_ms, 6),
        "mall_warm_l1_note": "every call on one layer instance (weights resident in the Infinity "
                             "Cache): not an HBM figure",
        "device_status": status,
    }


# measured into the default line beside the headline (batch-1 decode, 288 experts):
# the 512-expert layer (NVFP4, block-fp8, over expert slots), the batched decode call,
# the prefill chunk, the FP8 W8A8 projection (1 and 8192 tokens) and the extend
# attention over an NVFP4 cache
DEFAULT_ALSO = ",".join([
    "decode_e512_top10_shared", "decode_e512_top10_shared_fp8", "decode_e512_top10_shared_slots",
    "batched_decode_t32_hot64", "prefill_t8192", "fp8_linear_qkv_t1", "fp8_linear_qkv_t8192",
    "attn_extend_nvfp4_p4096_n512"])


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000,
                    help="calls per timed repetition")
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--reps", type=int, default=5, help="timed repetitions (median reported)")
    ap.add_argument("--workload", default="decode_e288_top8")
    ap.add_argument("--also", default=None,
                    help="comma-separated further decode workloads measured into the same line "
                         "(default: decode_e512_top10_shared with the default workload)")
    ap.add_argument("--instances", type=int, default=0,
                    help="distinct layer instances to cycle (0 = enough to exceed 4x the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--no-stream-probe", action="store_true")
    ap.add_argument("--no-mall-warm", action="store_true",
                    help="skip the Infinity-Cache-warm secondary decode figure (profiling runs)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run one plain elementwise copy (negation) of this many "
                         "MiB, as the known-size reference for HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library runs the layer on one MI355X and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        return 2
    if args.steps < 1 or args.reps < 1:
        print("--steps and --reps must be positive", file=sys.stderr)
        return 2

    import torch
    from nvfp4_mixture_experts_amd import ftmoe, synth

    ftmoe.ft_init(0)
    if args.workload in synth.LINEAR_WORKLOADS or args.workload.startswith("attn_"):
        m = (measure_attn(args, args.steps, args.reps) if args.workload.startswith("attn_")
             else measure_linear(args, synth.LINEAR_WORKLOADS[args.workload], args.steps,
                                 args.reps))
        out = {"metric": m["entry"] + ": calls/s", "value": m["value"], "unit": "calls/s",
               "n_gpus": 1, "steps": m["steps"], "warmup": args.warmup,
               "ms_per_step": m["ms_per_step"], "higher_is_better": True, "scaling": "weak",
               "vs_baseline": None, "dtype": "fp8" if "linear" in m["entry"] else "bf16",
               "data": "synthetic", "config": m["config"], "roofline": m["roofline"]}
        print(json.dumps(out), flush=True)
        return 0
    w = synth.WORKLOADS[args.workload]
    if w.tokens > 64:
        return run_prefill(args, w)
    also = args.also
    if also is None:
        also = DEFAULT_ALSO if args.workload == "decode_e288_top8" else ""
    also = [a for a in also.split(",") if a]

    main_m = measure_decode(args, w, args.steps, args.warmup, args.reps)
    extra = []
    for a in also:
        if a == "attn_extend_nvfp4_p4096_n512":
            extra.append(measure_attn(args, args.steps, args.reps))
        elif a.endswith("_slots"):
            extra.append(measure_decode(args, synth.WORKLOADS[a[:-len("_slots")]], args.steps,
                                        args.warmup, args.reps, variant="slots"))
        elif a in synth.LINEAR_WORKLOADS:
            extra.append(measure_linear(args, synth.LINEAR_WORKLOADS[a], args.steps, args.reps))
        elif synth.WORKLOADS[a].tokens > 64:
            extra.append(measure_prefill(args, synth.WORKLOADS[a], args.steps, args.warmup))
        else:
            extra.append(measure_decode(args, synth.WORKLOADS[a], args.steps, args.warmup,
                                        args.reps))
        print(f"measured {a}", file=sys.stderr, flush=True)
    out = {
        "metric": METRIC,
        "value": main_m["value"],
        "unit": "calls/s",
        "n_gpus": 1,
        "steps": main_m["steps"],
        "warmup": args.warmup,
        "ms_per_step": main_m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
    }
    for key in ("config", "roofline", "achieved_gbps", "hbm_peak_frac", "reps",
                "ms_per_step_reps", "wall_s_timed", "launch", "eager_ms_per_step",
                "mall_warm_l1_ms_per_step", "mall_warm_l1_note", "device_status"):
        out[key] = main_m[key]
    if extra:
        out["also"] = extra
    if not args.no_stream_probe:
        probe = stream_read_probe(torch.device("cuda:0"))
        probe["decode_frac_of_probe"] = round(main_m["achieved_gbps"] / probe["gbps"], 4)
        out["hbm_stream_probe"] = probe
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
