"""Benchmark of the NVFP4 MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]
                    [--variant w4a4|w4a16|mxfp4] [--mode graph|eager] [--no-configs]
                    [--no-linear] [--no-cpu]

A step is one pass of the whole layer path on one batch: global activation
scale, activation quantisation, permutation by expert, grouped GEMM1 with
SwiGLU and requantisation, grouped GEMM2 with the top-k weighted combine
(W4A16: permutation and the two GEMMs; MXFP4: block-scale quantisation,
permutation, the two GEMMs on the scaled FP4 matrix instruction).  Inputs
(activations, routing, prepared weights) are resident in HBM before timing
starts; routing and weight preparation are outside the step.  Several copies of the weights are rotated
between steps so the 256 MB Infinity Cache cannot serve repeats.

Prints one JSON line.  ``value`` is the tokens/s of the headline workload
(decode: T = 64, H = 2048, I = 768, E = 128, top-8) over exactly K timed
steps, after W warm-up steps; the K steps are one replay of a graph holding
K steps (default K = 200, W = 400: the device's clocks settle under
sustained load).  ``configs`` holds every other workload and variant (tiny,
decode W4A16, prefill, large_e, skew in both NVFP4 variants; decode, prefill
and large_e in OCP MXFP4; K/4 steps after W/4), each with its mean step, the
per-step median over 100 replays of its timed graph after 10 warm-up
replays, the per-stage breakdown, and the roofline figures of its dominant
kernel (GEMM1) measured with HIP events on the launch stream.  Layers whose
GEMMs run in two parts (the 512-expert layer: short experts and tall ones)
run the tall experts' part on a second stream inside the captured graph
(``"streams": 2``); the kernel figures time each GEMM whole on one stream.
``cpu_baseline`` is the FP64 oracle timed on the host cores on a bounded
sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_inputs  # noqa: E402
from nvfp4_block_scaled_03_amd import ops  # noqa: E402
from nvfp4_block_scaled_03_amd.profiling import (MxStep, build_layer, build_mx_weights,  # noqa: E402
                                                  mx_weight_copies, weight_copies)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense FP16/BF16 matrix peak
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 matrix peak
INFINITY_CACHE = 256 << 20
REPLAYS, REPLAY_WARMUP = 100, 10


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # Defaults: enough warm-up (two replays of the timed graph) for the
    # device's clocks to settle under sustained load before timing.
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=400)
    p.add_argument("--workload", default="decode", choices=moe_inputs.ORDER)
    p.add_argument("--variant", default="w4a4", choices=["w4a4", "w4a16", "mxfp4"])
    p.add_argument("--mode", default="graph", choices=["eager", "graph"])
    p.add_argument("--no-configs", action="store_true", help="skip the other workloads")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-linear", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dtype_label(variant):
    return {"w4a4": "nvfp4 codes, f16 matrix ops, f32 accumulate",
            "w4a16": "nvfp4 weights, bf16 activations, bf16 matrix ops, f32 accumulate",
            "mxfp4": "mxfp4 codes (E8M0 block scales), fp4 matrix ops, f32 accumulate"}[variant]


# Bytes per element of an operand held in each variant's format (codes and
# block scales, or bf16), and the matrix-unit peak its GEMMs run against.
def elem_bytes(variant):
    return {"w4a4": 0.5 + 1 / 16, "w4a16": 2.0, "mxfp4": 0.5 + 1 / 32}[variant]


def matrix_peak(variant):
    return MFMA_FP4_PEAK_TFLOPS if variant == "mxfp4" else MFMA_F16_PEAK_TFLOPS


# ---------------------------------------------------------------- CPU oracle
def _oracle_inputs(w, dev, n_tok):
    """Host copies of the sample: x, routing (the oracle's own router on the
    same logits), and expert weights fetched on demand."""
    from oracle import moe as omoe
    from oracle import routing as oroute
    x = moe_inputs.activations(w, device=dev).float().cpu().numpy().astype(np.float64)
    ids, tw = oroute.route_topk(moe_inputs.router_logits(w, device=dev).cpu().numpy(), w.topk)
    cache = {}

    def src(which):
        def get(e):
            if (which, e) not in cache:
                cache[(which, e)] = moe_inputs.expert_weight(w, which, e, device=dev).cpu().numpy()
            return cache[(which, e)]
        return get

    ew = omoe.ExpertWeights(src(13), src(2))
    used = set(int(e) for e in ids[:n_tok].reshape(-1)) | ({w.E} if w.shared else set())
    for e in used:              # offline weight quantisation: outside the timed scope, as on the GPU
        ew.quantized(13, e)
        ew.quantized(2, e)
    toks = np.arange(n_tok)
    g2 = omoe.calibrate_g2(x, ids, ew, w.E, w.I, w.shared, tokens=toks)
    return x, ids, tw, ew, toks, g2


def _time_oracle(w, x, ids, tw, ew, toks, g2, seconds, max_reps=1000):
    from oracle import moe as omoe
    reps, t0 = 0, time.perf_counter()
    while True:
        omoe.layer(x, ids, tw, ew, w.E, w.I, variant="w4a4", g2=g2, shared=w.shared, tokens=toks)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= max_reps:
            return reps, el


def cpu_baseline(w, dev, seconds):
    """The FP64 oracle (W4A4, same scope as the GPU step: global scale,
    quantisation, alignment, both GEMMs with SwiGLU and requantisation,
    combine) on a bounded sample of the workload's tokens, with every BLAS
    thread the process may use; then single-threaded on the tiny and decode
    layers."""
    import threadpoolctl
    info = threadpoolctl.threadpool_info()
    threads = max((i.get("num_threads", 1) for i in info), default=1)
    affinity = len(os.sched_getaffinity(0))
    n_tok = min(w.T, 16)
    x, ids, tw, ew, toks, g2 = _oracle_inputs(w, dev, n_tok)
    reps, el = _time_oracle(w, x, ids, tw, ew, toks, g2, seconds)
    flops = 6.0 * w.H * w.I * (n_tok * w.topk + (n_tok if w.shared else 0))
    res = {"value": n_tok * reps / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{n_tok} of {w.T} tokens of the {w.name} layer, W4A4, FP64 NumPy, "
                     f"{reps} repetitions in {el:.1f} s (weight quantisation excluded)",
           "gflops": round(flops * reps / el / 1e9, 2),
           "affinity_cores": affinity, "blas_threads": int(threads), "single_thread": []}
    with threadpoolctl.threadpool_limits(1):
        for name, n1, sec in (("tiny", 16, 3.0), ("decode", 4, 6.0)):
            w1 = moe_inputs.WORKLOADS[name]
            xi, idi, twi, ewi, ti, g2i = _oracle_inputs(w1, dev, n1)
            r1, e1 = _time_oracle(w1, xi, idi, twi, ewi, ti, g2i, sec)
            res["single_thread"].append({"workload": name, "tokens": n1, "reps": r1, "seconds": round(e1, 2),
                                         "tokens_per_s": round(n1 * r1 / e1, 3)})
    return res


# ---------------------------------------------------------------- GPU timing
def make_graphs(layer, x, ids, tw, copies, variant, out, per_graph):
    """One graph per weight copy (a single step) and one graph holding
    ``per_graph`` steps in sequence, cycling through the weight copies, as a
    model forward captures its consecutive layers in one graph (each replay
    boundary leaves the GPU idle for several microseconds)."""
    graphs = []
    for wc in copies:
        for _ in range(2):
            layer.forward(x, ids, tw, variant, out=out, weights=wc)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.forward(x, ids, tw, variant, out=out, weights=wc)
        graphs.append(g)
    multi = torch.cuda.CUDAGraph()
    with torch.cuda.graph(multi):
        for i in range(per_graph):
            layer.forward(x, ids, tw, variant, out=out, weights=copies[i % len(copies)])
    return graphs, multi


def upload_graph(g) -> bool:
    """Upload an instantiated graph's executable to the device before its
    first launch (hipGraphUpload), so that the timed replay does not pay the
    one-time upload of a few hundred kernel nodes.  Uses the HIP runtime
    already loaded in the process; returns False (nothing done) if that
    cannot be found or the call fails."""
    import ctypes
    try:
        path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line)
        hip = ctypes.CDLL(path)
        hip.hipGraphUpload.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipGraphUpload.restype = ctypes.c_int
        rc = hip.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        return rc == 0
    except (StopIteration, OSError, AttributeError, RuntimeError):
        return False


def time_steps(layer, x, ids, tw, copies, variant, steps, warmup, mode, graphs=None, multi=None,
               per_graph=0):
    """Mean wall time of one layer step (ms) over exactly ``steps`` steps
    (synchronised on both sides); graph mode replays the multi-step graph and
    the one-step graphs for a remainder."""
    out = torch.empty(x.shape[0], layer.d.H, dtype=torch.bfloat16, device=x.device)

    def run(i0, count):
        if multi is not None and count >= per_graph and i0 % len(copies) == 0:
            multi.replay()
            return per_graph
        if graphs:
            graphs[i0 % len(graphs)].replay()
        else:
            layer.forward(x, ids, tw, variant, out=out, weights=copies[i0 % len(copies)])
        return 1

    i = 0
    while i < warmup:
        i += run(i, warmup - i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while i < steps:
        i += run(i, steps - i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def replay_median(multi, per_graph, replays=REPLAYS, warmup=REPLAY_WARMUP):
    """Median (and spread) of the per-step time over ``replays`` replays of
    the multi-step graph, each bracketed by events on the current stream."""
    for _ in range(warmup):
        multi.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    ev[0].record()
    for i in range(replays):
        multi.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) / per_graph for i in range(replays))
    return {"replays": replays, "warmup_replays": warmup, "median_ms": round(statistics.median(per), 5),
            "p10_ms": round(per[replays // 10], 5), "p90_ms": round(per[(9 * replays) // 10], 5)}


def breakdown(layer, x, ids, tw, copies, variant, n=20):
    """Mean per-stage time (ms) of eager steps: front end (scale, quantise,
    align; W4A16: align), GEMM1, GEMM2 + combine; events on the launch stream."""
    out = torch.empty(x.shape[0], layer.d.H, dtype=torch.bfloat16, device=x.device)
    tot = np.zeros(3)
    for i in range(n + 3):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        ev[0].record()
        layer.forward(x, ids, tw, variant, out=out, weights=copies[i % len(copies)], marks=ev[1:])
        torch.cuda.synchronize()
        if i >= 3:
            tot += [ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2]), ev[2].elapsed_time(ev[3])]
    t = tot / n
    return {"front_ms": round(t[0], 5), "gemm1_ms": round(t[1], 5), "gemm2_combine_ms": round(t[2], 5),
            "eager_step_ms": round(float(t.sum()), 5)}


def time_gemm1(layer, x, ids, tw, copies, variant, n=50):
    """Mean duration (ms) of GEMM1 launched back to back, bracketed by events
    recorded on the stream the kernels run on."""
    layer.forward(x, ids, tw, variant, weights=copies[0])
    for i in range(5):
        layer.gemm1(variant, copies[i % len(copies)], x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        layer.gemm1(variant, copies[i % len(copies)], x)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def measured_traffic(workload: str, variant: str, kernel: str = "grouped_gemm1_swiglu"):
    """HBM bytes per call of ``kernel`` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or None
    when there is none for this workload and variant or the kernel sources
    changed since it was taken."""
    from nvfp4_block_scaled_03_amd import profiling
    suffix = {"w4a4": "", "w4a16": "_w4a16", "mxfp4": "_mxfp4"}[variant]
    path = os.path.join(ROOT, "profiles", f"{kernel}{suffix}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    t = profiling.read_traffic(path)
    family = "mxfp4" if variant == "mxfp4" else "nvfp4"
    if t.get("sources_sha256_16") != profiling.sources_hash(family):
        return None
    return int(float(t["bytes_per_call"]))


def measure(w, built, variant, steps, warmup, mode, mx_weights=None):
    """Step time (mean over ``steps``), replay median, breakdown and GEMM1
    roofline for one workload and variant (``mx_weights``: the prepared MXFP4
    weights, variant mxfp4)."""
    d, x, ids, tw, wq, g2 = built
    P = w.pairs
    al = ops.moe_align(d, ids)
    rows_per_expert = np.diff(al.offsets.cpu().numpy())
    touched = int((rows_per_expert > 0).sum())
    block = 32 if variant == "mxfp4" else 16
    wbytes13 = (2 * w.I * w.H) // 2 + (2 * w.I * w.H) // block
    wbytes2 = (w.I * w.H) // 2 + (w.I * w.H) // block
    n_copies = min(8, max(1, math.ceil(4 * INFINITY_CACHE / max(1, touched * (wbytes13 + wbytes2)))))
    # Layers whose GEMMs run in two parts (short and tall experts) overlap
    # them on a second stream.
    side = torch.cuda.Stream()
    if variant == "mxfp4":
        copies = mx_weight_copies(mx_weights, n_copies)
        layer = MxStep(d, mx_weights, x.device, side_stream=side)
    else:
        copies = weight_copies(wq, n_copies)
        layer = ops.MoELayer(d, wq, g2, device=x.device, side_stream=side)
    inner = layer.layer if variant == "mxfp4" else layer
    streams = 2 if inner.side is not None and (variant != "w4a4" or inner.decoded_copies) else 1
    out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=x.device)
    graphs = multi = None
    # The timed steps are one replay of a graph of that many steps.
    per_graph = max(steps, len(copies))
    uploaded = False
    if mode == "graph":
        graphs, multi = make_graphs(layer, x, ids, tw, copies, variant, out, per_graph)
        uploaded = upload_graph(multi)
    ms = time_steps(layer, x, ids, tw, copies, variant, steps, warmup, mode, graphs, multi, per_graph)
    rep = replay_median(multi, per_graph) if multi is not None else None
    bd = breakdown(layer, x, ids, tw, copies, variant)
    g1_ms = time_gemm1(layer, x, ids, tw, copies, variant)
    g1_flops = 2.0 * P * (2 * w.I) * w.H
    eb = elem_bytes(variant)
    g1_bytes = int(touched * wbytes13 + w.T * w.H * eb + P * w.I * eb)
    peak = matrix_peak(variant)
    decode_like = P / max(1, w.n_experts) < 64
    if decode_like:
        ach = g1_bytes / (g1_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w.name, variant)}
    else:
        ach = g1_flops / (g1_ms * 1e-3) / 1e12
        # (traffic: the HBM bytes the matrix-bound kernel moved, for the
        # record; its roofline is the matrix peak)
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": measured_traffic(w.name, variant)}
    roof.update({"kernel": "grouped_gemm1_swiglu" + {"w4a4": "", "w4a16": "_w4a16", "mxfp4": "_mxfp4"}[variant],
                 "kernel_ms": round(g1_ms, 5), "algorithmic_bytes": g1_bytes,
                 "algorithmic_flops": g1_flops})
    layer_flops = moe_inputs.flops(w)
    layer_bytes = moe_inputs.touched_bytes(w, rows_per_expert, block)
    med = rep["median_ms"] if rep else ms
    rec = {
        "workload": w.name, **w.describe(), "variant": variant, "mode": mode,
        "experts_touched": touched, "weight_copies": len(copies),
        "steps_per_graph": per_graph if mode == "graph" else 1, "graph_uploaded": uploaded, "streams": streams,
        "steps": steps, "ms_per_step": round(ms, 5), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
        "layer_tflops": round(layer_flops / (ms * 1e-3) / 1e12, 2),
        "layer_gbs": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
        "layer_hbm_frac": round(layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_mfma_frac": round(layer_flops / (ms * 1e-3) / 1e12 / peak, 4),
        "median_tokens_per_s": round(w.T / (med * 1e-3), 1),
        "breakdown": bd, "roofline": roof,
    }
    if rep:
        rec["replay"] = rep
    del graphs, multi, layer, copies
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


# ---------------------------------------------------------------- dense linear
LINEAR_N, LINEAR_K = 34816, 5120          # the pages' per-GEMM shape (27B gate_up)
LINEAR_MS = (1, 16, 64, 256, 1024, 4096)


def _graph_us(fn, reps):
    """Average microseconds of fn(i) for i in range(reps), replayed from one graph."""
    fn(0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(reps):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def linear_sweep(dev, copies=3, reps=10):
    """Dense linear y = x W^T across batch sizes M: NVFP4 W4A4 (quantisation
    of x included), NVFP4 W4A16, and OCP MXFP4 (x quantised in the call, the
    codes fed to the scaled FP4 matrix instruction), each timed as ``reps``
    calls replayed from one graph with weight copies rotated past the
    Infinity Cache."""
    N, K = LINEAR_N, LINEAR_K
    g = torch.Generator(device=dev).manual_seed(21)
    w = 0.02 * torch.randn(N, K, generator=g, device=dev)
    lw = ops.quantize_linear_weight(w)
    mw = ops.quantize_mx_weight(w)
    del w
    ws = [lw] + [ops.LinearWeight(lw.prep.clone(), lw.g.clone(), N, K) for _ in range(copies - 1)]
    mws = [mw] + [ops.MxLinearWeight(mw.prep.clone(), N, K) for _ in range(copies - 1)]
    peaks = {"w4a4": MFMA_F16_PEAK_TFLOPS, "w4a16": MFMA_F16_PEAK_TFLOPS, "mxfp4": MFMA_FP4_PEAK_TFLOPS}
    w_bytes = {"w4a4": N * K * 0.5625, "w4a16": N * K * 0.5625, "mxfp4": N * K * (0.5 + 1 / 32)}
    rows = []
    for M in LINEAR_MS:
        x = torch.randn(M, K, generator=g, device=dev).to(torch.bfloat16)
        row = {"M": M}
        for variant in ("w4a4", "w4a16", "mxfp4"):
            out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            if variant == "mxfp4":
                work = ops.mx_linear_workspace(M, N, K, dev)
                fn = lambda i: ops.mx_linear(x, mws[i % copies], out=out, ws=work)
            else:
                work = ops.linear_workspace(M, N, K, variant == "w4a4", dev)
                fn = lambda i: ops.linear(x, ws[i % copies], variant, out=out, ws=work)
            for i in range(copies):
                fn(i)
            us = _graph_us(fn, reps)
            flops = 2.0 * M * N * K
            nbytes = w_bytes[variant] + M * K * 2 + M * N * 2
            row[f"{variant}_us"] = round(us, 2)
            row[f"{variant}_tflops"] = round(flops / us / 1e6, 1)
            row[f"{variant}_gbs"] = round(nbytes / us / 1e3, 1)
            row[f"{variant}_hbm_frac"] = round(nbytes / us / 1e3 / HBM_PEAK_GBS, 3)
            row[f"{variant}_mfma_frac"] = round(flops / us / 1e6 / peaks[variant], 3)
        row["w4a16_over_w4a4"] = round(row["w4a16_us"] / row["w4a4_us"], 2)
        rows.append(row)
    return {"shape": {"N": N, "K": K}, "weight_copies": copies, "calls_per_graph": reps,
            "w4a4_includes": "global scale + quantisation of x + tile plan + GEMM",
            "w4a16_includes": "tile plan + GEMM",
            "mxfp4_includes": "MXFP4 quantisation of x + GEMM (mfma_frac against the FP4 peak)",
            "rows": rows}


# ---------------------------------------------------------------- main
# The other workloads and variants reported next to the headline line (the
# five workload shapes in both NVFP4 variants, three of them in MXFP4, and one
# GPU's share of the prefill layer under 8-way expert parallelism).
# Prefill reuses the decode layer's weights (the same expert shape).
OTHER_CONFIGS = [("decode", "w4a16"), ("decode", "mxfp4"), ("tiny", "w4a4"), ("prefill", "w4a4"),
                 ("prefill", "w4a16"), ("prefill", "mxfp4"), ("large_e", "w4a4"), ("large_e", "w4a16"),
                 ("large_e", "mxfp4"), ("skew", "w4a4"), ("skew", "w4a16"), ("ep8_share", "w4a4")]


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; --gpus must be 1 (no second GPU is used)"}))
        sys.exit(2)
    dev = torch.device("cuda:0")
    w = moe_inputs.WORKLOADS[a.workload]
    log(f"[bench] building {w.name} layer ({a.variant}, {a.mode})")
    built = {w.name: build_layer(w, dev)}
    mx = {}                     # prepared MXFP4 weights per workload (prefill shares decode's)

    def mx_weights(name):
        key = "decode" if name == "prefill" else name
        if key not in mx:
            log(f"[bench] building {key} MXFP4 weights")
            mx[key] = build_mx_weights(moe_inputs.WORKLOADS[key], dev)
        return mx[key]

    log(f"[bench] timing {a.steps} steps")
    m = measure(w, built[w.name], a.variant, a.steps, a.warmup, a.mode,
                mx_weights(w.name) if a.variant == "mxfp4" else None)
    res = {
        "metric": "NVFP4 MoE layer tokens/s (30B-A3B expert shape)",
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_label(a.variant),
        "data": "synthetic (seeded), random-init weights",
        "config": {"workload": w.name, **w.describe(), "variant": a.variant, "mode": a.mode,
                   "experts_touched": m["experts_touched"], "weight_copies": m["weight_copies"],
                   "steps_per_graph": m["steps_per_graph"], "graph_uploaded": m["graph_uploaded"],
                   "streams": m["streams"]},
        "layer_tflops": m["layer_tflops"], "layer_gbs": m["layer_gbs"],
        "layer_hbm_frac": m["layer_hbm_frac"],
        "roofline": m["roofline"],
        "replay": m.get("replay"), "breakdown": m["breakdown"],
    }
    if not a.no_configs:
        res["configs"] = {}
        for name, variant in OTHER_CONFIGS:
            if name == a.workload and variant == a.variant:
                continue
            wc = moe_inputs.WORKLOADS[name]
            if name not in built:
                # drop layers no later config uses (bounded device memory)
                for k in [k for k in built if k not in ("decode",) and k != name]:
                    del built[k]
                    mx.pop(k, None)
                torch.cuda.empty_cache()
                reuse = built["decode"][4] if name == "prefill" and "decode" in built else None
                log(f"[bench] building {name} layer")
                built[name] = build_layer(wc, dev, weights=reuse)
            log(f"[bench] {name} {variant}")
            steps = max(5, a.steps // 4)
            res["configs"][f"{name}_{variant}"] = measure(
                wc, built[name], variant, steps, max(3, a.warmup // 4), a.mode,
                mx_weights(name) if variant == "mxfp4" else None)
    built.clear()
    mx.clear()
    torch.cuda.empty_cache()
    if not a.no_linear:
        log("[bench] dense linear M sweep")
        res["linear"] = linear_sweep(dev)
    if not a.no_cpu:
        log("[bench] cpu baseline")
        res["cpu_baseline"] = cpu_baseline(w, dev, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
