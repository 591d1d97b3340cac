"""Programs and summaries for rocprofv3 runs of the hot path.

    python -m nvfp4_block_scaled_03_amd.profiling gemm1|gemm2 [--workload decode]
            [--variant w4a4] [--reps 5]
        Launch GEMM1 (or GEMM2 + combine) of the named layer ``reps`` times,
        weight copies rotated as in bench.py (the kernel to collect counters
        for).
    python -m nvfp4_block_scaled_03_amd.profiling layer [--workload decode]
            [--variant w4a4] [--steps 20]
        Eager passes of the whole layer (the program of a kernel trace).
    python -m nvfp4_block_scaled_03_amd.profiling copy [--mib 1024] [--reps 3]
        A plain device-to-device copy of a known size (counter calibration:
        FETCH_SIZE / WRITE_SIZE per dispatch against the bytes really moved).
    python -m nvfp4_block_scaled_03_amd.profiling counters --csv A.csv [B.csv ...]
        --kernel-re RE --title T --command C > profiles/<kernel>_<workload>_counters.txt
        Mean value per dispatch of every counter collected for the kernels
        matching RE, and the matrix-unit and VALU busy fractions derived
        from them (rocprofv3's MfmaUtil and VALUBusy formulas).
    python -m nvfp4_block_scaled_03_amd.profiling traffic --fetch F.csv --write W.csv
        --copy-fetch CF.csv --copy-write CW.csv --mib 1024 --kernel NAME --workload decode
        [--req R.csv] --command "..." > profiles/<kernel>_<workload>_traffic.txt
        Summarise two counter runs of the kernel and two of the copy into the
        HBM bytes per launch (counter readings scaled by the copy calibration)
        and record the hash of the kernel sources the counters belong to.

bench.py reads the traffic summary and reports it only while the sources
still hash to the recorded value (a changed kernel invalidates the counters).
``build_layer`` and ``weight_copies`` build the benchmark's layers (bench.py
and the profiling programs above share them).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
# Sources whose change invalidates recorded counters of the GEMM kernels, by
# kernel family (the NVFP4 GEMMs, the MXFP4 GEMMs).
HASHED = {"nvfp4": ["csrc/gemm.hip", "csrc/common.h", "csrc/launch.h", "csrc/prep.hip"],
          "mxfp4": ["csrc/mx.hip", "csrc/mx.h", "csrc/common.h", "csrc/launch.h"]}


def sources_hash(family: str = "nvfp4") -> str:
    h = hashlib.sha256()
    for rel in HASHED[family]:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _per_dispatch(path: str, counter: str, name_re: str):
    """Mean counter value per dispatch (KiB for *_SIZE) of kernels matching name_re."""
    vals = defaultdict(float)
    names = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or not re.search(name_re, r["Kernel_Name"]):
                continue
            d = r["Dispatch_Id"]
            vals[d] += float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
    if not vals:
        raise SystemExit(f"no {counter} rows for /{name_re}/ in {path}")
    return sum(vals.values()) / len(vals), len(vals), sorted(set(names.values()))


def read_traffic(path: str):
    """Parse a traffic summary: dict with bytes_per_call, fetch/write bytes, hash."""
    out = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"\s*([a-z0-9_]+)\s*=\s*(\S+)", line)
            if m:
                out[m.group(1)] = m.group(2)
    return out


def build_layer(w, dev, weights=None):
    """Inputs and prepared NVFP4 weights of workload ``w`` on device ``dev``:
    (dims, x, topk_ids, topk_w, ExpertWeights, g2).  Routing by the library's
    router; weights quantised and prepared by the library, expert group by
    expert group (bounded FP32 memory); g2 calibrated from the layer's own
    W4A16 intermediate.  ``weights`` reuses prepared weights of the same
    expert shape instead of building new ones."""
    import torch
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import moe_inputs
    from nvfp4_block_scaled_03_amd import ops
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    x = moe_inputs.activations(w, device=dev)
    logits = moe_inputs.router_logits(w, device=dev)
    ids, tw = ops.route_topk(logits, w.topk)
    if weights is None:
        S = w.n_experts
        chunk = max(1, min(S, (8 << 30) // (4 * 3 * w.I * w.H)))
        parts = []
        for s0 in range(0, S, chunk):
            sel = range(s0, min(S, s0 + chunk))
            w13 = moe_inputs.expert_weights(w, 13, device=dev, experts=sel)
            w2 = moe_inputs.expert_weights(w, 2, device=dev, experts=sel)
            g13 = ops.global_scale(w13, batches=len(sel))
            q13, sf13 = ops.quantize(w13.reshape(-1, w.H), g13, rows_per_g=2 * w.I)
            g2w = ops.global_scale(w2, batches=len(sel))
            q2, sf2 = ops.quantize(w2.reshape(-1, w.I), g2w, rows_per_g=w.H)
            parts.append((q13.view(len(sel), 2 * w.I, -1), sf13.view(len(sel), 2 * w.I, -1), g13,
                          q2.view(len(sel), w.H, -1), sf2.view(len(sel), w.H, -1), g2w))
            del w13, w2
        cat = [torch.cat([p[i] for p in parts]) for i in range(6)]
        del parts
        prep13 = ops.prep_weights(d, 13, cat[0], cat[1])
        prep2 = ops.prep_weights(d, 2, cat[3], cat[4])
        empty = torch.empty(0, dtype=torch.uint8, device=dev)
        weights = ops.ExpertWeights(empty, empty, cat[2], empty, empty, cat[5], prep13, prep2)
        del cat
    g2 = ops.calibrate_g2(d, x, ids, weights)
    torch.cuda.synchronize()
    return d, x, ids, tw, weights, g2


def weight_copies(wq, n):
    """``n`` independent copies of the prepared weights (the first is ``wq``),
    rotated between steps so that the Infinity Cache cannot serve repeats."""
    from nvfp4_block_scaled_03_amd import ops
    out = [wq]
    for _ in range(n - 1):
        out.append(ops.ExpertWeights(wq.q13, wq.sf13, wq.g13.clone(), wq.q2, wq.sf2, wq.g2.clone(),
                                     wq.prep13.clone(), wq.prep2.clone()))
    return out


def build_mx_weights(w, dev):
    """OCP MXFP4 expert weights of workload ``w`` (the same FP32 source
    weights as build_layer), quantised and prepared by the library expert
    group by expert group (bounded FP32 memory, under 2^31 elements a call)."""
    import torch
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import moe_inputs
    from nvfp4_block_scaled_03_amd import ops
    d = ops.dims(w.T, w.topk, w.E, w.H, w.I, w.shared)
    S, I, H = w.n_experts, w.I, w.H
    chunk = max(1, min(S, (8 << 30) // (4 * 3 * I * H), ((1 << 31) - 1) // (2 * I * H)))
    u8 = dict(dtype=torch.uint8, device=dev)
    q13, e13 = torch.empty(S * 2 * I, H // 2, **u8), torch.empty(S * 2 * I, H // 32, **u8)
    q2, e2 = torch.empty(S * H, I // 2, **u8), torch.empty(S * H, I // 32, **u8)
    for s0 in range(0, S, chunk):
        s1 = min(S, s0 + chunk)
        sel = range(s0, s1)
        w13 = moe_inputs.expert_weights(w, 13, device=dev, experts=sel)
        ops.mx_quantize(w13.reshape(-1, H), q=q13[s0 * 2 * I:s1 * 2 * I], ex=e13[s0 * 2 * I:s1 * 2 * I])
        del w13
        w2 = moe_inputs.expert_weights(w, 2, device=dev, experts=sel)
        ops.mx_quantize(w2.reshape(-1, I), q=q2[s0 * H:s1 * H], ex=e2[s0 * H:s1 * H])
        del w2
    wq = ops.MxExpertWeights(ops.prep_mx_expert_weights(d, 13, q13, e13),
                             ops.prep_mx_expert_weights(d, 2, q2, e2))
    torch.cuda.synchronize()
    return wq


def mx_weight_copies(wq, n):
    """``n`` independent copies of prepared MXFP4 expert weights."""
    from nvfp4_block_scaled_03_amd import ops
    return [wq] + [ops.MxExpertWeights(wq.prep13.clone(), wq.prep2.clone()) for _ in range(n - 1)]


class MxStep:
    """The MXFP4 layer behind the calls of ops.MoELayer (forward, gemm1,
    gemm2 with a variant argument), so that timing and profiling code drives
    both layers alike."""

    def __init__(self, d, weights, dev, side_stream=None):
        from nvfp4_block_scaled_03_amd import ops
        self.d = d
        self.layer = ops.MxMoELayer(d, weights, device=dev, side_stream=side_stream)

    def forward(self, x, ids, tw, variant, out=None, weights=None, marks=None):
        return self.layer.forward(x, ids, tw, out=out, weights=weights, marks=marks)

    def gemm1(self, variant, weights, x):
        self.layer.gemm1(weights)

    def gemm2(self, variant, out, weights, tw):
        self.layer.gemm2(out, tw, weights)


def make_layer(w, dev, variant, built=None):
    """(layer, weight copies, dims, x, ids, tw) of workload ``w`` for one
    variant; the NVFP4 variants share one build, mxfp4 builds its weights."""
    from nvfp4_block_scaled_03_amd import ops
    d, x, ids, tw, wq, g2 = built if built is not None else build_layer(w, dev)
    if variant == "mxfp4":
        mq = build_mx_weights(w, dev)
        return MxStep(d, mq, dev), mx_weight_copies(mq, 4), d, x, ids, tw
    return ops.MoELayer(d, wq, g2, device=dev), weight_copies(wq, 4), d, x, ids, tw


def _cmd_gemm(a):
    """Launch one GEMM of the named layer ``reps`` times (weight copies
    rotated), after one full layer pass has filled its inputs."""
    import torch
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import moe_inputs
    dev = torch.device("cuda:0")
    w = moe_inputs.WORKLOADS[a.workload]
    layer, copies, d, x, ids, tw = make_layer(w, dev, a.variant)
    out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev)
    layer.forward(x, ids, tw, a.variant, out=out)
    torch.cuda.synchronize()
    for i in range(a.reps):
        if a.cmd == "gemm1":
            layer.gemm1(a.variant, copies[i % len(copies)], x)
        else:
            layer.gemm2(a.variant, out, copies[i % len(copies)], tw)
    torch.cuda.synchronize()
    print(f"{a.cmd} {a.workload} {a.variant}: {a.reps} launches", flush=True)


def _cmd_layer(a):
    """``steps`` eager layer passes of the named workload (weight copies
    rotated): the program behind the kernel-trace summaries."""
    import torch
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import moe_inputs
    dev = torch.device("cuda:0")
    w = moe_inputs.WORKLOADS[a.workload]
    layer, copies, d, x, ids, tw = make_layer(w, dev, a.variant)
    out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev)
    for i in range(a.steps):
        layer.forward(x, ids, tw, a.variant, out=out, weights=copies[i % len(copies)])
    torch.cuda.synchronize()
    print(f"layer {a.workload} {a.variant}: {a.steps} steps", flush=True)


def _cmd_copy(a):
    import torch
    n = a.mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(a.reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy {a.mib} MiB x {a.reps}", flush=True)


def _cmd_traffic(a):
    # A call of some GEMMs is several launches (short and tall experts):
    # per-call figures are per-dispatch means times launches per call.
    f_kib, n_f, names = _per_dispatch(a.fetch, "FETCH_SIZE", a.kernel_re)
    w_kib, n_w, _ = _per_dispatch(a.write, "WRITE_SIZE", a.kernel_re)
    f_kib *= a.launches_per_call
    w_kib *= a.launches_per_call
    cf_kib, _, cnames = _per_dispatch(a.copy_fetch, "FETCH_SIZE", a.copy_re)
    cw_kib, _, _ = _per_dispatch(a.copy_write, "WRITE_SIZE", a.copy_re)
    moved = float(a.mib << 20)
    f_scale = moved / (cf_kib * 1024.0)
    w_scale = moved / (cw_kib * 1024.0)
    fetch_b = f_kib * 1024.0 * f_scale
    write_b = w_kib * 1024.0 * w_scale
    print(f"# HBM traffic of {a.kernel} ({a.workload}), rocprofv3 counter collection")
    print(f"# command (kernel, per counter): {a.command}")
    print(f"# calibration: plain copy of {a.mib} MiB (reads {a.mib} MiB, writes {a.mib} MiB)")
    print(f"# kernels matched: {'; '.join(n[:90] for n in names)}")
    print(f"# copy kernel: {'; '.join(n[:90] for n in cnames)}")
    print(f"kernel = {a.kernel}")
    print(f"workload = {a.workload}")
    print(f"dispatches_fetch = {n_f}")
    print(f"dispatches_write = {n_w}")
    print(f"launches_per_call = {a.launches_per_call}")
    print(f"fetch_size_kib_per_call = {f_kib:.1f}")
    print(f"write_size_kib_per_call = {w_kib:.1f}")
    print(f"copy_fetch_size_kib = {cf_kib:.1f}")
    print(f"copy_write_size_kib = {cw_kib:.1f}")
    print(f"fetch_scale = {f_scale:.4f}")
    print(f"write_scale = {w_scale:.4f}")
    print(f"fetch_bytes_per_call = {fetch_b:.0f}")
    print(f"write_bytes_per_call = {write_b:.0f}")
    print(f"bytes_per_call = {fetch_b + write_b:.0f}")
    if a.req:
        # Cross-check of the fetch calibration: HBM read requests by size.
        sizes = {"TCC_EA0_RDREQ_32B_sum": 32, "TCC_EA0_RDREQ_64B_sum": 64, "TCC_EA0_RDREQ_128B_sum": 128}
        req_b = sum(_per_dispatch(a.req, c, a.kernel_re)[0] * b for c, b in sizes.items())
        print(f"read_bytes_by_request_size = {req_b:.0f}")
    print(f"family = {a.family}")
    print(f"sources_sha256_16 = {sources_hash(a.family)}")


def _cmd_stats(a):
    rows = []
    with open(a.csv) as f:
        for r in csv.DictReader(f):
            if a.exclude_re and re.search(a.exclude_re, r["Name"]):
                continue
            rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]), float(r["AverageNs"]),
                         float(r["MinNs"]), float(r["MaxNs"])))
    total = sum(r[2] for r in rows)
    print(f"# rocprofv3 --kernel-trace --stats summary ({a.title})")
    print(f"# command: {a.command}")
    if a.exclude_re:
        print(f"# kernels matching /{a.exclude_re}/ left out (input and weight preparation)")
    print(f"# {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'share':>6}  kernel")
    for name, calls, tot, avg, mn, mx in sorted(rows, key=lambda r: -r[2])[:a.top]:
        short = re.sub(r"\(anonymous namespace\)::", "", name)
        short = re.sub(r"\(nvfp4::KParams\)|\(.*$", "", short)[:100]
        print(f"  {calls:6d} {avg / 1e3:9.2f} {mn / 1e3:9.2f} {mx / 1e3:9.2f} {100 * tot / total:5.1f}%  {short}")


def _cmd_counters(a):
    vals = defaultdict(lambda: defaultdict(float))
    names = set()
    for path in a.csv:
        with open(path) as f:
            for r in csv.DictReader(f):
                if not re.search(a.kernel_re, r["Kernel_Name"]):
                    continue
                vals[r["Counter_Name"]][(path, r["Dispatch_Id"])] += float(r["Counter_Value"])
                names.add(re.sub(r"\(.*$", "", r["Kernel_Name"]))
    if not vals:
        raise SystemExit(f"no counter rows for /{a.kernel_re}/")
    mean = {c: sum(d.values()) / len(d) for c, d in vals.items()}
    print(f"# rocprofv3 counters per dispatch ({a.title})")
    print(f"# command: {a.command}")
    print(f"# kernels matched: {', '.join(sorted(names))[:160]}")
    for c in sorted(mean):
        print(f"{c} = {mean[c]:.6g}   # {len(vals[c])} dispatches")
    gui = mean.get("GRBM_GUI_ACTIVE")
    if gui:
        # rocprofv3's derived metrics (its counter list): MfmaUtil =
        # sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) * SIMD_NUM),
        # VALUBusy = sum(SQ_ACTIVE_INST_VALU) / CU_NUM / max(GRBM_GUI_ACTIVE).
        # The CSV holds each counter summed over its dimensions, so the
        # per-XCC maximum of GRBM_GUI_ACTIVE is taken as the sum over the 8
        # XCCs / 8.  MI355X: 256 CUs, 1024 SIMDs.
        cycles = gui / 8.0
        print(f"gui_cycles_per_xcc = {cycles:.6g}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
            print(f"mfma_util = {mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (cycles * 1024):.4f}")
        if "SQ_ACTIVE_INST_VALU" in mean:
            print(f"valu_busy = {mean['SQ_ACTIVE_INST_VALU'] / 256 / cycles:.4f}")
        if "SQ_LDS_BANK_CONFLICT" in mean:
            print(f"lds_bank_conflict_cycles_per_cu_over_gui = "
                  f"{mean['SQ_LDS_BANK_CONFLICT'] / 256 / cycles:.4f}")


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    for name in ("gemm1", "gemm2"):
        g = sub.add_parser(name)
        g.add_argument("--workload", default="decode")
        g.add_argument("--variant", default="w4a4", choices=["w4a4", "w4a16", "mxfp4"])
        g.add_argument("--reps", type=int, default=5)
    ly = sub.add_parser("layer")
    ly.add_argument("--workload", default="decode")
    ly.add_argument("--variant", default="w4a4", choices=["w4a4", "w4a16", "mxfp4"])
    ly.add_argument("--steps", type=int, default=20)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=3)
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--mib", type=int, default=1024)
    t.add_argument("--kernel", default="grouped_gemm1_swiglu")
    t.add_argument("--kernel-re", dest="kernel_re", default=r"grouped_gemm_stream\d?_kernel<0, 0,")
    t.add_argument("--copy-re", dest="copy_re", default=r"copy|Copy")
    t.add_argument("--workload", default="decode")
    t.add_argument("--command", default="")
    t.add_argument("--req", default="", help="counter CSV of TCC_EA0_RDREQ_{32B,64B,128B}_sum")
    t.add_argument("--family", default="nvfp4", choices=sorted(HASHED))
    t.add_argument("--launches-per-call", dest="launches_per_call", type=int, default=1)
    co = sub.add_parser("counters")
    co.add_argument("--csv", nargs="+", required=True)
    co.add_argument("--kernel-re", dest="kernel_re", required=True)
    co.add_argument("--title", default="")
    co.add_argument("--command", default="")
    st = sub.add_parser("stats")
    st.add_argument("--csv", required=True)
    st.add_argument("--title", default="")
    st.add_argument("--command", default="")
    st.add_argument("--top", type=int, default=16)
    st.add_argument("--exclude-re", dest="exclude_re", default="")
    a = p.parse_args(argv)
    {"gemm1": _cmd_gemm, "gemm2": _cmd_gemm, "layer": _cmd_layer, "copy": _cmd_copy,
     "traffic": _cmd_traffic, "stats": _cmd_stats, "counters": _cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
