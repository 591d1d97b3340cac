"""Benchmark of the NVFP4 MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]
                    [--variant w4a4|w4a16] [--mode graph|eager] [--no-cpu]

A step is one pass of the whole layer path on one batch: global activation
scale, activation quantisation, permutation by expert, grouped GEMM1 with
SwiGLU and requantisation, grouped GEMM2 with the top-k weighted combine
(W4A16: permutation and the two GEMMs).  Inputs (activations, routing,
prepared weights) are resident in HBM before timing starts; routing and weight
preparation are outside the step.  Several copies of the weights are rotated
between steps so the 256 MB Infinity Cache cannot serve repeats.

Prints one JSON line: throughput in tokens/s, the dominant kernel's roofline
figures measured with HIP events inside the timed region, and the CPU oracle's
throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_inputs  # noqa: E402
from nvfp4_block_scaled_03_amd import ops  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense FP16/BF16 matrix peak
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 matrix peak
INFINITY_CACHE = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode", choices=moe_inputs.ORDER)
    p.add_argument("--variant", default="w4a4", choices=["w4a4", "w4a16"])
    p.add_argument("--mode", default="graph", choices=["eager", "graph"])
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-linear", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_layer(w, dev):
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    x = moe_inputs.activations(w, device=dev)
    logits = moe_inputs.router_logits(w, device=dev)
    ids, tw = ops.route_topk(logits, w.topk)
    # Quantise the weights expert-group by expert-group to bound FP32 memory.
    S = w.n_experts
    chunk = max(1, min(S, (8 << 30) // (4 * 3 * w.I * w.H)))
    parts = []
    for s0 in range(0, S, chunk):
        sel = range(s0, min(S, s0 + chunk))
        sub = ops.dims(w.T, w.topk, len(sel), w.H, w.I, 0)
        w13 = moe_inputs.expert_weights(w, 13, device=dev, experts=sel)
        w2 = moe_inputs.expert_weights(w, 2, device=dev, experts=sel)
        g13 = ops.global_scale(w13, batches=len(sel))
        q13, sf13 = ops.quantize(w13.reshape(-1, w.H), g13, rows_per_g=2 * w.I)
        g2w = ops.global_scale(w2, batches=len(sel))
        q2, sf2 = ops.quantize(w2.reshape(-1, w.I), g2w, rows_per_g=w.H)
        parts.append((q13.view(len(sel), 2 * w.I, -1), sf13.view(len(sel), 2 * w.I, -1), g13,
                      q2.view(len(sel), w.H, -1), sf2.view(len(sel), w.H, -1), g2w))
        del w13, w2, sub
    cat = [torch.cat([p[i] for p in parts]) for i in range(6)]
    del parts
    prep13 = ops.prep_weights(d, 13, cat[0], cat[1])
    prep2 = ops.prep_weights(d, 2, cat[3], cat[4])
    empty = torch.empty(0, dtype=torch.uint8, device=dev)
    wq = ops.ExpertWeights(empty, empty, cat[2], empty, empty, cat[5], prep13, prep2)
    del cat
    g2 = ops.calibrate_g2(d, x, ids, wq)
    torch.cuda.synchronize()
    return d, x, ids, tw, wq, g2


def weight_copies(wq, n):
    out = [wq]
    for _ in range(n - 1):
        out.append(ops.ExpertWeights(wq.q13, wq.sf13, wq.g13.clone(), wq.q2, wq.sf2, wq.g2.clone(),
                                     wq.prep13.clone(), wq.prep2.clone()))
    return out


def cpu_baseline(w, dev, ids, tw, seconds):
    """The FP64 oracle on a bounded sample of the workload's tokens (host cores)."""
    from oracle import moe as omoe
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) \
            if threadpoolctl.threadpool_info() else 1
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    n_tok = min(w.T, 16)
    toks = np.arange(n_tok)
    x = moe_inputs.activations(w, device=dev).float().cpu().numpy().astype(np.float64)
    ids_np, tw_np = ids.cpu().numpy(), tw.cpu().numpy()
    cache13, cache2 = {}, {}

    def src13(e):
        if e not in cache13:
            cache13[e] = moe_inputs.expert_weight(w, 13, e, device=dev).cpu().numpy()
        return cache13[e]

    def src2(e):
        if e not in cache2:
            cache2[e] = moe_inputs.expert_weight(w, 2, e, device=dev).cpu().numpy()
        return cache2[e]

    ew = omoe.ExpertWeights(src13, src2)
    # Offline weight quantisation is outside the timed scope, as on the GPU.
    used = set(int(e) for e in ids_np[:n_tok].reshape(-1)) | ({w.E} if w.shared else set())
    for e in used:
        ew.quantized(13, e)
        ew.quantized(2, e)
    g2 = np.float32(1e-3)
    reps, t0 = 0, time.perf_counter()
    while True:
        omoe.layer(x, ids_np, tw_np, ew, w.E, w.I, variant="w4a4", g2=g2, shared=w.shared,
                   tokens=toks)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    return {"value": n_tok * reps / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_tok} of {w.T} tokens of the {w.name} layer, W4A4, FP64 NumPy, "
                      f"{reps} repetitions in {el:.1f} s (weight quantisation excluded)"}


def time_steps(layer, x, ids, tw, copies, variant, steps, warmup, mode):
    """Mean wall time of one layer step (ms) over ``steps`` steps.

    Graph mode captures the steps of all weight copies in one graph, one
    complete step per copy in sequence, as a model forward captures its
    consecutive layers; a remainder of steps runs from one-step graphs."""
    out = torch.empty(x.shape[0], layer.d.H, dtype=torch.bfloat16, device=x.device)
    graphs, multi = [], None
    if mode == "graph":
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
            for wc in copies:
                layer.forward(x, ids, tw, variant, out=out, weights=wc)

    def run(i0, count):
        """Steps i0 .. i0 + count - 1; returns how many ran."""
        if multi is not None and count >= len(copies) and i0 % len(copies) == 0:
            multi.replay()
            return len(copies)
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


def measured_traffic(workload: str, variant: str):
    """HBM bytes per GEMM1 launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or None when there
    is none for this workload or the kernel sources changed since it was taken."""
    from nvfp4_block_scaled_03_amd import profiling
    if variant != "w4a4":
        return None
    path = os.path.join(ROOT, "profiles", f"grouped_gemm1_swiglu_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    t = profiling.read_traffic(path)
    if t.get("sources_sha256_16") != profiling.sources_hash():
        return None
    return int(float(t["bytes_per_launch"]))


def measure(w, d, x, ids, tw, wq, g2, a, steps, warmup):
    """Step time, GEMM1 time and the derived figures for one batch shape."""
    P = w.pairs
    al = ops.moe_align(d, ids)
    rows_per_expert = np.diff(al.offsets.cpu().numpy())
    touched = int((rows_per_expert > 0).sum())
    wbytes13 = (2 * w.I * w.H) // 2 + (2 * w.I * w.H) // 16
    wbytes2 = (w.I * w.H) // 2 + (w.I * w.H) // 16
    n_copies = max(1, math.ceil(4 * INFINITY_CACHE / max(1, touched * (wbytes13 + wbytes2))))
    copies = weight_copies(wq, min(n_copies, 8))
    layer = ops.MoELayer(d, wq, g2, device=x.device)
    ms = time_steps(layer, x, ids, tw, copies, a.variant, steps, warmup, a.mode)
    g1_ms = time_gemm1(layer, x, ids, tw, copies, a.variant)
    g1_flops = 2.0 * P * (2 * w.I) * w.H
    g1_bytes = touched * wbytes13 + w.T * (w.H // 2 + w.H // 16) + P * (w.I // 2 + w.I // 16)
    decode_like = P / max(1, w.n_experts) < 64
    if decode_like:
        ach = g1_bytes / (g1_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(w.name, a.variant)}
    else:
        ach = g1_flops / (g1_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None}
    roof.update({"kernel": "grouped_gemm1_swiglu" + ("" if a.variant == "w4a4" else "_w4a16"),
                 "kernel_ms": round(g1_ms, 5), "algorithmic_bytes": int(g1_bytes),
                 "algorithmic_flops": g1_flops})
    layer_flops = moe_inputs.flops(w)
    layer_bytes = moe_inputs.touched_bytes(w, rows_per_expert)
    return {
        "ms": ms, "tokens_per_s": w.T / (ms * 1e-3), "touched": touched,
        "copies": len(copies), "roofline": roof,
        "layer_tflops": round(layer_flops / (ms * 1e-3) / 1e12, 2),
        "layer_gbs": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
        "layer_hbm_frac": round(layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_mfma_frac": round(layer_flops / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
    }


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


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; --gpus must be 1"}))
        sys.exit(2)
    dev = torch.device("cuda:0")
    w = moe_inputs.WORKLOADS[a.workload]
    log(f"[bench] building {w.name} layer ({a.variant}, {a.mode})")
    d, x, ids, tw, wq, g2 = build_layer(w, dev)
    log(f"[bench] timing {a.steps} steps")
    m = measure(w, d, x, ids, tw, wq, g2, a, a.steps, a.warmup)
    res = {
        "metric": "NVFP4 MoE layer tokens/s (30B-A3B expert shape)",
        "value": round(m["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(m["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 codes, f16 matrix ops, f32 accumulate" if a.variant == "w4a4"
                 else "nvfp4 weights, bf16 activations, bf16 matrix ops, f32 accumulate",
        "data": "synthetic (seeded), random-init weights",
        "config": {"workload": w.name, **w.describe(), "variant": a.variant, "mode": a.mode,
                   "experts_touched": m["touched"], "weight_copies": m["copies"],
                   "steps_per_graph": m["copies"] if a.mode == "graph" else 1},
        "layer_tflops": m["layer_tflops"], "layer_gbs": m["layer_gbs"],
        "layer_hbm_frac": m["layer_hbm_frac"],
        "roofline": m["roofline"],
    }
    if a.workload == "decode" and not a.no_prefill:
        # The prefill-shaped batch (T = 4096) on the same layer weights.
        wp = moe_inputs.WORKLOADS["prefill"]
        log("[bench] prefill batch on the same layer")
        dp = ops.dims(wp.T, wp.topk, wp.E, wp.H, wp.I, wp.shared)
        xp = moe_inputs.activations(wp, device=dev)
        idp, twp = ops.route_topk(moe_inputs.router_logits(wp, device=dev), wp.topk)
        g2p = ops.calibrate_g2(dp, xp, idp, wq)
        mp = measure(wp, dp, xp, idp, twp, wq, g2p, a, max(5, a.steps // 4), max(2, a.warmup // 2))
        res["prefill"] = {"T": wp.T, "tokens_per_s": round(mp["tokens_per_s"], 1),
                          "ms_per_step": round(mp["ms"], 5), "layer_tflops": mp["layer_tflops"],
                          "layer_mfma_frac": mp["layer_mfma_frac"], "roofline": mp["roofline"]}
    if a.workload == "decode" and not a.no_linear:
        log("[bench] dense linear M sweep")
        res["linear"] = linear_sweep(dev)
    if not a.no_cpu:
        log("[bench] cpu baseline")
        res["cpu_baseline"] = cpu_baseline(w, dev, ids, tw, a.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
