"""Thin torch binding over the C ABI: argument marshalling only.

Every step runs in the HIP library; torch provides device memory and the
current stream.  Names follow include/nvfp4_moe.h.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib
from ._lib import NVFP4_BF16, NVFP4_F32, Dims, call


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return NVFP4_BF16
    if t.dtype == torch.float32:
        return NVFP4_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def dims(T: int, topk: int, E: int, H: int, I: int, shared: int = 0) -> Dims:
    return Dims(T, topk, E, H, I, shared)


# ---------------------------------------------------------------- codec
def global_scale(x: torch.Tensor, batches: int = 1, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """g[b] = fl32(max |x[b]| / 2688) over ``batches`` equal contiguous slices."""
    _need_cuda(x)
    x = x.contiguous()
    n = x.numel() // batches if batches else 0
    g = out if out is not None else torch.empty(batches, dtype=torch.float32, device=x.device)
    lib = _lib.load()
    wsb = lib.nvfp4_global_scale_workspace_size(batches, n)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=x.device)
    call("nvfp4_global_scale", _p(x), _dtype_code(x), batches, n, _p(g), _p(ws), wsb, _stream())
    return g


def quantize(x: torch.Tensor, g: torch.Tensor, rows_per_g: Optional[int] = None,
             q: Optional[torch.Tensor] = None, sf: Optional[torch.Tensor] = None,
             deq: Optional[torch.Tensor] = None):
    """NVFP4-encode the rows of ``x`` [rows, K]: (codes [rows, K/2], scales [rows, K/16]).
    ``deq`` (float16 [rows, K]) optionally receives the exact decoded values."""
    _need_cuda(x, g)
    K = x.shape[-1]
    x2 = x.reshape(-1, K)
    if x2.stride(-1) != 1:
        x2 = x2.contiguous()
    rows = x2.shape[0]
    if q is None:
        q = torch.empty(rows, K // 2, dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty(rows, K // 16, dtype=torch.uint8, device=x.device)
    call("nvfp4_quantize", _p(x2), _dtype_code(x2), rows, K, x2.stride(0), _p(g),
         rows if rows_per_g is None else rows_per_g, _p(q), _p(sf), _p(deq), _stream())
    return q, sf


# ---------------------------------------------------------------- routing
def route_topk(logits: torch.Tensor, k: int):
    _need_cuda(logits)
    logits = logits.contiguous().float()
    T, E = logits.shape
    ids = torch.empty(T, k, dtype=torch.int32, device=logits.device)
    w = torch.empty(T, k, dtype=torch.float32, device=logits.device)
    call("moe_route_topk", _p(logits), T, E, k, _p(ids), _p(w), _stream())
    return ids, w


@dataclasses.dataclass
class Alignment:
    offsets: torch.Tensor
    sorted_pair: torch.Tensor
    inv_pos: torch.Tensor
    plan: torch.Tensor
    workspace: torch.Tensor


def alloc_alignment(d: Dims, device) -> Alignment:
    lib = _lib.load()
    P = d.T * d.topk + d.shared * d.T
    return Alignment(
        offsets=torch.empty(d.E + d.shared + 1, dtype=torch.int32, device=device),
        sorted_pair=torch.empty(max(P, 1), dtype=torch.int32, device=device),
        inv_pos=torch.empty(max(P, 1), dtype=torch.int32, device=device),
        plan=torch.empty(lib.moe_align_plan_size(ctypes.byref(d)) // 4, dtype=torch.int32,
                         device=device),
        workspace=torch.empty(max(lib.moe_align_workspace_size(ctypes.byref(d)), 16),
                              dtype=torch.uint8, device=device))


def moe_align(d: Dims, topk_ids: torch.Tensor, al: Optional[Alignment] = None) -> Alignment:
    _need_cuda(topk_ids)
    al = al or alloc_alignment(d, topk_ids.device)
    call("moe_align", ctypes.byref(d), _p(topk_ids.contiguous()), _p(al.offsets),
         _p(al.sorted_pair), _p(al.inv_pos), _p(al.plan), _p(al.workspace),
         al.workspace.numel(), _stream())
    return al


def route_and_align(d: Dims, logits: torch.Tensor, al: Optional[Alignment] = None):
    """Router (top-k + softmax over the selection) and moe_align in one call:
    (topk_ids int32 [T, topk], topk_w float32 [T, topk], Alignment)."""
    _need_cuda(logits)
    al = al or alloc_alignment(d, logits.device)
    ids = torch.empty(max(d.T, 1), d.topk, dtype=torch.int32, device=logits.device)
    wts = torch.empty(max(d.T, 1), d.topk, dtype=torch.float32, device=logits.device)
    call("moe_route_and_align", ctypes.byref(d), _p(logits.contiguous().float()), _p(ids), _p(wts),
         _p(al.offsets), _p(al.sorted_pair), _p(al.inv_pos), _p(al.plan), _p(al.workspace),
         al.workspace.numel(), _stream())
    return ids[:d.T], wts[:d.T], al


def quantize_and_align(d: Dims, x: torch.Tensor, topk_ids: torch.Tensor, al: Optional[Alignment] = None,
                       deq: Optional[torch.Tensor] = None):
    """Global scale, NVFP4 quantisation and moe_align of bf16 ``x`` [T, H] in
    one call: (g, codes, scales, Alignment); ``deq`` optionally receives the
    exact f16 values."""
    _need_cuda(x, topk_ids)
    al = al or alloc_alignment(d, x.device)
    g = torch.empty(1, dtype=torch.float32, device=x.device)
    q = torch.empty(max(d.T, 1), d.H // 2, dtype=torch.uint8, device=x.device)
    sf = torch.empty(max(d.T, 1), d.H // 16, dtype=torch.uint8, device=x.device)
    wsb = _lib.load().nvfp4_global_scale_workspace_size(1, d.T * d.H)
    gs_ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=x.device)
    call("moe_quantize_and_align", ctypes.byref(d), _p(x.contiguous()), _p(g), _p(gs_ws), wsb,
         _p(q), _p(sf), _p(deq), _p(topk_ids.contiguous()), _p(al.offsets), _p(al.sorted_pair),
         _p(al.inv_pos), _p(al.plan), _p(al.workspace), al.workspace.numel(), _stream())
    return g, q, sf, al


def mx_quantize_and_align(d: Dims, x: torch.Tensor, topk_ids: torch.Tensor, al: Optional[Alignment] = None):
    """OCP MXFP4 quantisation and moe_align of bf16 ``x`` [T, H] in one call:
    (codes [T, H/2], E8M0 bytes [T, H/32], Alignment)."""
    _need_cuda(x, topk_ids)
    al = al or alloc_alignment(d, x.device)
    q = torch.empty(max(d.T, 1), d.H // 2, dtype=torch.uint8, device=x.device)
    ex = torch.empty(max(d.T, 1), d.H // 32, dtype=torch.uint8, device=x.device)
    call("moe_mxfp4_quantize_and_align", ctypes.byref(d), _p(x.contiguous()), _p(q), _p(ex),
         _p(topk_ids.contiguous()), _p(al.offsets), _p(al.sorted_pair), _p(al.inv_pos), _p(al.plan),
         _p(al.workspace), al.workspace.numel(), _stream())
    return q, ex, al


def scale_and_align(d: Dims, x: torch.Tensor, topk_ids: torch.Tensor, al: Optional[Alignment] = None):
    """Activation global scale of bf16 ``x`` [T, H] and moe_align in one call: (g, Alignment)."""
    _need_cuda(x, topk_ids)
    al = al or alloc_alignment(d, x.device)
    g = torch.empty(1, dtype=torch.float32, device=x.device)
    wsb = _lib.load().nvfp4_global_scale_workspace_size(1, d.T * d.H)
    gs_ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=x.device)
    call("moe_scale_and_align", ctypes.byref(d), _p(x.contiguous()), _p(g), _p(gs_ws), wsb,
         _p(topk_ids.contiguous()), _p(al.offsets), _p(al.sorted_pair), _p(al.inv_pos), _p(al.plan),
         _p(al.workspace), al.workspace.numel(), _stream())
    return g, al, gs_ws


# ---------------------------------------------------------------- weights
def prep_weights(d: Dims, which: int, q: torch.Tensor, sf: torch.Tensor) -> torch.Tensor:
    _need_cuda(q, sf)
    n = _lib.load().nvfp4_prep_weights_size(ctypes.byref(d), which)
    prep = torch.empty(n, dtype=torch.uint8, device=q.device)
    call("nvfp4_prep_weights", ctypes.byref(d), which, _p(q.contiguous()), _p(sf.contiguous()),
         _p(prep), _stream())
    return prep


@dataclasses.dataclass
class ExpertWeights:
    """NVFP4 expert weights of one layer: canonical codes/scales, per-matrix
    global scales, and the library's streaming layout."""
    q13: torch.Tensor    # uint8 [S, 2I, H/2]
    sf13: torch.Tensor   # uint8 [S, 2I, H/16]
    g13: torch.Tensor    # f32 [S]
    q2: torch.Tensor     # uint8 [S, H, I/2]
    sf2: torch.Tensor    # uint8 [S, H, I/16]
    g2: torch.Tensor     # f32 [S]
    prep13: torch.Tensor
    prep2: torch.Tensor


def quantize_expert_weights(d: Dims, w13: torch.Tensor, w2: torch.Tensor,
                            keep_canonical: bool = True) -> ExpertWeights:
    """Quantise FP32 expert weights (w13 [S, 2I, H], w2 [S, H, I]) on the GPU:
    one global scale per expert matrix, then block quantisation and prep."""
    S = d.E + d.shared
    assert w13.shape == (S, 2 * d.I, d.H) and w2.shape == (S, d.H, d.I)
    g13 = global_scale(w13, batches=S)
    q13, sf13 = quantize(w13.reshape(S * 2 * d.I, d.H), g13, rows_per_g=2 * d.I)
    g2 = global_scale(w2, batches=S)
    q2, sf2 = quantize(w2.reshape(S * d.H, d.I), g2, rows_per_g=d.H)
    q13 = q13.view(S, 2 * d.I, d.H // 2)
    sf13 = sf13.view(S, 2 * d.I, d.H // 16)
    q2 = q2.view(S, d.H, d.I // 2)
    sf2 = sf2.view(S, d.H, d.I // 16)
    prep13 = prep_weights(d, 13, q13, sf13)
    prep2 = prep_weights(d, 2, q2, sf2)
    if not keep_canonical:
        empty = torch.empty(0, dtype=torch.uint8, device=w13.device)
        q13 = sf13 = q2 = sf2 = empty
    return ExpertWeights(q13, sf13, g13, q2, sf2, g2, prep13, prep2)


# ---------------------------------------------------------------- GEMMs
def gemm1_w4a4(d: Dims, a1_q, a1_sf, g1, al: Alignment, w: ExpertWeights, g2, a2_q=None, a2_sf=None,
               a1_deq=None, a2_deq=None):
    """GEMM1 + SwiGLU + requantisation.  ``a1_deq`` (the decoded copy from
    ``quantize``) is read instead of the codes when given; ``a2_deq``
    optionally receives the decoded copy of a2."""
    P = d.T * d.topk + d.shared * d.T
    dev = g1.device
    a2_q = a2_q if a2_q is not None else torch.empty(max(P, 1), d.I // 2, dtype=torch.uint8, device=dev)
    a2_sf = a2_sf if a2_sf is not None else torch.empty(max(P, 1), d.I // 16, dtype=torch.uint8, device=dev)
    call("grouped_gemm1_swiglu", ctypes.byref(d), _p(a1_q), _p(a1_sf), _p(a1_deq), _p(g1),
         _p(al.sorted_pair), _p(al.offsets), _p(al.plan), _p(w.prep13), _p(w.g13), _p(g2),
         _p(a2_q), _p(a2_sf), _p(a2_deq), _stream())
    return a2_q, a2_sf


def gemm1_w4a16(d: Dims, x, al: Alignment, w: ExpertWeights, a2=None):
    P = d.T * d.topk + d.shared * d.T
    a2 = a2 if a2 is not None else torch.empty(max(P, 1), d.I, dtype=torch.bfloat16, device=x.device)
    call("grouped_gemm1_swiglu_w4a16", ctypes.byref(d), _p(x), _p(al.sorted_pair), _p(al.offsets),
         _p(al.plan), _p(w.prep13), _p(w.g13), _p(a2), _stream())
    return a2


def gemm_workspace(d: Dims, device) -> torch.Tensor:
    n = _lib.load().grouped_gemm_workspace_size(ctypes.byref(d))
    return torch.empty(max(n // 4, 4), dtype=torch.float32, device=device)


def gemm2_w4a4(d: Dims, a2_q, a2_sf, g2, al: Alignment, topk_w, w: ExpertWeights,
               out_dtype=torch.bfloat16, out=None, ws=None, a2_deq=None):
    dev = g2.device
    out = out if out is not None else torch.empty(d.T, d.H, dtype=out_dtype, device=dev)
    ws = ws if ws is not None else gemm_workspace(d, dev)
    call("grouped_gemm2_combine", ctypes.byref(d), _p(a2_q), _p(a2_sf), _p(a2_deq), _p(g2),
         _p(al.offsets), _p(al.inv_pos), _p(al.plan), _p(topk_w), _p(w.prep2), _p(w.g2), _p(out),
         _dtype_code(out), _p(ws), ws.numel() * 4, _stream())
    return out


def gemm2_w4a4_noalloc(d: Dims, a2_q, a2_sf, g2, al: Alignment, topk_w, w: ExpertWeights,
                       out: torch.Tensor, a2_deq=None):
    """grouped_gemm2_combine_noalloc: GEMM2 + combine with the library's
    static scratch instead of a workspace (``out`` is caller-allocated)."""
    call("grouped_gemm2_combine_noalloc", ctypes.byref(d), _p(a2_q), _p(a2_sf), _p(a2_deq), _p(g2),
         _p(al.offsets), _p(al.inv_pos), _p(al.plan), _p(topk_w), _p(w.prep2), _p(w.g2), _p(out),
         _dtype_code(out), _stream())
    return out


def gemm2_w4a16(d: Dims, a2, al: Alignment, topk_w, w: ExpertWeights, out_dtype=torch.bfloat16,
                out=None, ws=None):
    dev = a2.device
    out = out if out is not None else torch.empty(d.T, d.H, dtype=out_dtype, device=dev)
    ws = ws if ws is not None else gemm_workspace(d, dev)
    call("grouped_gemm2_combine_w4a16", ctypes.byref(d), _p(a2), _p(al.offsets), _p(al.inv_pos),
         _p(al.plan), _p(topk_w), _p(w.prep2), _p(w.g2), _p(out), _dtype_code(out), _p(ws),
         ws.numel() * 4, _stream())
    return out


# ---------------------------------------------------------------- dense linear
class LinearWeight:
    """An NVFP4 weight W [N, K] prepared for nvfp4_linear*."""

    def __init__(self, prep: torch.Tensor, g: torch.Tensor, N: int, K: int):
        self.prep, self.g, self.N, self.K = prep, g, N, K


def prepare_linear_weight(w_q: torch.Tensor, w_sf: torch.Tensor, g: torch.Tensor) -> LinearWeight:
    """From canonical NVFP4 (codes [N, K/2], scales [N, K/16], global scale)."""
    N, K = w_q.shape[0], w_q.shape[1] * 2
    d = dims(1, 1, 1, N, K, 0)
    prep = prep_weights(d, 2, w_q.reshape(1, N, K // 2), w_sf.reshape(1, N, K // 16))
    return LinearWeight(prep, g.reshape(1).float(), N, K)


def quantize_linear_weight(w: torch.Tensor) -> LinearWeight:
    """FP32 W [N, K] -> global scale, NVFP4 quantisation on the GPU, prep."""
    g = global_scale(w)
    q, sf = quantize(w.contiguous().float(), g)
    return prepare_linear_weight(q, sf, g)


def linear_workspace(M: int, N: int, K: int, w4a4: bool, device) -> torch.Tensor:
    n = _lib.load().nvfp4_linear_workspace_size(M, N, K, int(w4a4))
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def linear(x: torch.Tensor, w: LinearWeight, variant: str = "w4a4", out_dtype=torch.bfloat16,
           out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [M, N] = x [M, K] W^T (bf16 x; W4A4 quantises x, W4A16 uses it as is)."""
    _need_cuda(x)
    M = x.shape[0]
    w4a4 = variant == "w4a4"
    out = out if out is not None else torch.empty(M, w.N, dtype=out_dtype, device=x.device)
    ws = ws if ws is not None else linear_workspace(M, w.N, w.K, w4a4, x.device)
    call("nvfp4_linear" if w4a4 else "nvfp4_linear_w4a16", _p(x.contiguous()), M, w.N, w.K, _p(w.prep),
         _p(w.g), _p(out), _dtype_code(out), _p(ws), ws.numel(), _stream())
    return out


# ---------------------------------------------------------------- OCP MXFP4
def mx_quantize(x: torch.Tensor, q: Optional[torch.Tensor] = None, ex: Optional[torch.Tensor] = None):
    """MXFP4-encode the rows of ``x`` [rows, K]: (codes [rows, K/2], E8M0 bytes [rows, K/32])."""
    _need_cuda(x)
    K = x.shape[-1]
    x2 = x.reshape(-1, K)
    if x2.stride(-1) != 1:
        x2 = x2.contiguous()
    rows = x2.shape[0]
    q = q if q is not None else torch.empty(rows, K // 2, dtype=torch.uint8, device=x.device)
    ex = ex if ex is not None else torch.empty(rows, K // 32, dtype=torch.uint8, device=x.device)
    call("mxfp4_quantize", _p(x2), _dtype_code(x2), rows, K, x2.stride(0), _p(q), _p(ex), _stream())
    return q, ex


class MxLinearWeight:
    """An MXFP4 weight W [N, K] prepared for mxfp4_linear."""

    def __init__(self, prep: torch.Tensor, N: int, K: int):
        self.prep, self.N, self.K = prep, N, K


def prepare_mx_weight(w_q: torch.Tensor, w_ex: torch.Tensor) -> MxLinearWeight:
    """From canonical MXFP4 (codes [N, K/2], exponent bytes [N, K/32])."""
    _need_cuda(w_q, w_ex)
    N, K = w_q.shape[0], w_q.shape[1] * 2
    n = _lib.load().mxfp4_prep_weights_size(N, K)
    prep = torch.empty(max(n, 16), dtype=torch.uint8, device=w_q.device)
    call("mxfp4_prep_weights", N, K, _p(w_q.contiguous()), _p(w_ex.contiguous()), _p(prep), _stream())
    return MxLinearWeight(prep, N, K)


def quantize_mx_weight(w: torch.Tensor) -> MxLinearWeight:
    """FP32 or bf16 W [N, K] -> MXFP4 quantisation on the GPU, prep."""
    q, ex = mx_quantize(w.contiguous())
    return prepare_mx_weight(q, ex)


def mx_linear_workspace(M: int, N: int, K: int, device) -> torch.Tensor:
    n = _lib.load().mxfp4_linear_workspace_size(M, N, K)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def mx_linear(x: torch.Tensor, w: MxLinearWeight, out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None,
              ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [M, N] = Q(x) W^T, x bf16 [M, K] quantised to MXFP4 in the call."""
    _need_cuda(x)
    M = x.shape[0]
    out = out if out is not None else torch.empty(M, w.N, dtype=out_dtype, device=x.device)
    ws = ws if ws is not None else mx_linear_workspace(M, w.N, w.K, x.device)
    call("mxfp4_linear", _p(x.contiguous()), M, w.N, w.K, _p(w.prep), _p(out), _dtype_code(out), _p(ws),
         ws.numel(), _stream())
    return out


# ---------------------------------------------------------------- MXFP4 layer
@dataclasses.dataclass
class MxExpertWeights:
    """OCP MXFP4 expert weights prepared for the grouped MXFP4 GEMMs."""
    prep13: torch.Tensor
    prep2: torch.Tensor


def prep_mx_expert_weights(d: Dims, which: int, q: torch.Tensor, ex: torch.Tensor) -> torch.Tensor:
    _need_cuda(q, ex)
    n = _lib.load().mxfp4_prep_expert_weights_size(ctypes.byref(d), which)
    prep = torch.empty(n, dtype=torch.uint8, device=q.device)
    call("mxfp4_prep_expert_weights", ctypes.byref(d), which, _p(q.contiguous()), _p(ex.contiguous()),
         _p(prep), _stream())
    return prep


def quantize_mx_expert_weights(d: Dims, w13: torch.Tensor, w2: torch.Tensor) -> MxExpertWeights:
    """FP32 expert weights (w13 [S, 2I, H], w2 [S, H, I]) -> MXFP4 on the GPU -> prep."""
    S = d.E + d.shared
    # mxfp4_quantize takes fewer than 2^31 elements per call: expert groups
    per = max(1, ((1 << 31) - 1) // (2 * d.I * d.H))
    q13 = torch.empty(S * 2 * d.I, d.H // 2, dtype=torch.uint8, device=w13.device)
    e13 = torch.empty(S * 2 * d.I, d.H // 32, dtype=torch.uint8, device=w13.device)
    q2 = torch.empty(S * d.H, d.I // 2, dtype=torch.uint8, device=w13.device)
    e2 = torch.empty(S * d.H, d.I // 32, dtype=torch.uint8, device=w13.device)
    for s0 in range(0, S, per):
        s1 = min(S, s0 + per)
        mx_quantize(w13[s0:s1].reshape(-1, d.H), q=q13[s0 * 2 * d.I:s1 * 2 * d.I], ex=e13[s0 * 2 * d.I:s1 * 2 * d.I])
        mx_quantize(w2[s0:s1].reshape(-1, d.I), q=q2[s0 * d.H:s1 * d.H], ex=e2[s0 * d.H:s1 * d.H])
    return MxExpertWeights(prep_mx_expert_weights(d, 13, q13, e13), prep_mx_expert_weights(d, 2, q2, e2))


PART_ALL, PART_SHORT, PART_TALL, PART_COMBINE = 0, 1, 2, 3


def _side_stream_if_parts(d: Dims, side_stream):
    """The side stream to use, or None when these dims run the GEMMs whole."""
    if side_stream is None or not _lib.load().grouped_gemm_runs_in_parts(ctypes.byref(d)):
        return None
    return side_stream


def _run_gemms(side, gemm1, gemm2, marks=None):
    """GEMM1 then GEMM2 + combine of one layer; ``gemm1(part, stream)`` and
    ``gemm2(part, stream)`` launch one part.  With a side stream, the tall
    experts' part of both GEMMs runs there (each part's GEMM2 reads only the
    rows its GEMM1 wrote) while the short experts' part runs on the current
    stream, which then waits for the side stream and runs the combine.  The
    events make the fork and the join part of a captured graph too."""
    main = torch.cuda.current_stream()
    s = ctypes.c_void_p(main.cuda_stream)
    if side is None:
        gemm1(PART_ALL, s)
        if marks:
            marks[1].record()
        gemm2(PART_ALL, s)
    else:
        side.wait_stream(main)
        ss = ctypes.c_void_p(side.cuda_stream)
        gemm1(PART_TALL, ss)
        gemm2(PART_TALL, ss)
        gemm1(PART_SHORT, s)
        if marks:
            marks[1].record()
        gemm2(PART_SHORT, s)
        main.wait_stream(side)
        gemm2(PART_COMBINE, s)
    if marks:
        marks[2].record()


class MxMoELayer:
    """One OCP MXFP4 expert layer with its intermediates preallocated (a call
    launches kernels only): mxfp4_quantize, moe_align,
    grouped_gemm1_swiglu_mxfp4, grouped_gemm2_combine_mxfp4."""

    def __init__(self, d: Dims, weights: MxExpertWeights, device="cuda", side_stream=None):
        """``side_stream``: a second stream for layers that run their GEMMs
        in two parts (``grouped_gemm_runs_in_parts``): the tall experts' part
        then runs on it beside the short experts' part."""
        self.d, self.w = d, weights
        dev = torch.device(device)
        self.side = _side_stream_if_parts(d, side_stream)
        P = d.T * d.topk + d.shared * d.T
        self.a1_q = torch.empty(max(d.T, 1), d.H // 2, dtype=torch.uint8, device=dev)
        self.a1_e = torch.empty(max(d.T, 1), d.H // 32, dtype=torch.uint8, device=dev)
        self.al = alloc_alignment(d, dev)
        self.a2_q = torch.empty(max(P, 1), d.I // 2, dtype=torch.uint8, device=dev)
        self.a2_e = torch.empty(max(P, 1), d.I // 32, dtype=torch.uint8, device=dev)
        self.ws = gemm_workspace(d, dev)

    def forward(self, x, topk_ids, topk_w, out=None, out_dtype=torch.bfloat16, weights=None, marks=None):
        d, w, s = self.d, weights or self.w, _stream()
        if out is None:
            out = torch.empty(d.T, d.H, dtype=out_dtype, device=x.device)
        call("moe_mxfp4_quantize_and_align", ctypes.byref(d), _p(x), _p(self.a1_q), _p(self.a1_e), _p(topk_ids),
             _p(self.al.offsets), _p(self.al.sorted_pair), _p(self.al.inv_pos), _p(self.al.plan),
             _p(self.al.workspace), self.al.workspace.numel(), s)
        if marks:
            marks[0].record()
        g1 = lambda part, st: call(
            "grouped_gemm1_swiglu_mxfp4_part", ctypes.byref(d), _p(self.a1_q), _p(self.a1_e),
            _p(self.al.sorted_pair), _p(self.al.offsets), _p(self.al.plan), _p(w.prep13),
            _p(self.a2_q), _p(self.a2_e), part, st)
        g2 = lambda part, st: call(
            "grouped_gemm2_combine_mxfp4_part", ctypes.byref(d), _p(self.a2_q), _p(self.a2_e),
            _p(self.al.offsets), _p(self.al.inv_pos), _p(self.al.plan), _p(topk_w), _p(w.prep2),
            _p(out), _dtype_code(out), _p(self.ws), self.ws.numel() * 4, part, st)
        _run_gemms(self.side, g1, g2, marks)
        return out

    def gemm1(self, weights=None):
        d, w = self.d, weights or self.w
        call("grouped_gemm1_swiglu_mxfp4", ctypes.byref(d), _p(self.a1_q), _p(self.a1_e),
             _p(self.al.sorted_pair), _p(self.al.offsets), _p(self.al.plan), _p(w.prep13),
             _p(self.a2_q), _p(self.a2_e), _stream())

    def gemm2(self, out, topk_w, weights=None):
        d, w = self.d, weights or self.w
        call("grouped_gemm2_combine_mxfp4", ctypes.byref(d), _p(self.a2_q), _p(self.a2_e),
             _p(self.al.offsets), _p(self.al.inv_pos), _p(self.al.plan), _p(topk_w), _p(w.prep2),
             _p(out), _dtype_code(out), _p(self.ws), self.ws.numel() * 4, _stream())


# ---------------------------------------------------------------- the layer
class MoELayer:
    """One NVFP4 expert layer with all intermediates preallocated, so that a
    call launches kernels only (and can be captured in a HIP graph)."""

    def __init__(self, d: Dims, weights: ExpertWeights, g2: torch.Tensor, device="cuda",
                 decoded_copies: Optional[bool] = None, side_stream=None):
        """``decoded_copies``: W4A4 keeps exact f16 copies of a1 and a2 next to
        their codes and the GEMMs read those instead of decoding the codes.
        None (default) asks the library which is faster for these dims (the
        copies pay off for tall tiles, not for decode-sized batches).
        ``side_stream``: as for MxMoELayer (W4A4 splits only with the copies)."""
        self.d = d
        self.w = weights
        self.g2 = g2
        P = d.T * d.topk + d.shared * d.T
        self.P = P
        dev = torch.device(device)
        lib = _lib.load()
        self.g1 = torch.empty(1, dtype=torch.float32, device=dev)
        wsb = lib.nvfp4_global_scale_workspace_size(1, d.T * d.H)
        self.gs_ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)  # zero once
        self.gs_ws_bytes = wsb
        self.a1_q = torch.empty(max(d.T, 1), d.H // 2, dtype=torch.uint8, device=dev)
        self.a1_sf = torch.empty(max(d.T, 1), d.H // 16, dtype=torch.uint8, device=dev)
        self.al = alloc_alignment(d, dev)
        self.a2_q = torch.empty(max(P, 1), d.I // 2, dtype=torch.uint8, device=dev)
        self.a2_sf = torch.empty(max(P, 1), d.I // 16, dtype=torch.uint8, device=dev)
        self.a2_bf16 = torch.empty(max(P, 1), d.I, dtype=torch.bfloat16, device=dev)
        self.a1_deq = self.a2_deq = None
        if decoded_copies is None:
            decoded_copies = bool(lib.grouped_gemm_prefers_decoded(ctypes.byref(d)))
        self.decoded_copies = decoded_copies
        if decoded_copies:
            self.a1_deq = torch.empty(max(d.T, 1), d.H, dtype=torch.float16, device=dev)
            self.a2_deq = torch.empty(max(P, 1), d.I, dtype=torch.float16, device=dev)
        self.ws = gemm_workspace(d, dev)
        self.side = _side_stream_if_parts(d, side_stream)

    def _gemm1_w4a4(self, w, s):
        d = self.d
        call("grouped_gemm1_swiglu", ctypes.byref(d), _p(self.a1_q), _p(self.a1_sf), _p(self.a1_deq),
             _p(self.g1), _p(self.al.sorted_pair), _p(self.al.offsets), _p(self.al.plan),
             _p(w.prep13), _p(w.g13), _p(self.g2), _p(self.a2_q), _p(self.a2_sf), _p(self.a2_deq), s)

    def _gemm2_w4a4(self, w, tw, out, s):
        d = self.d
        call("grouped_gemm2_combine", ctypes.byref(d), _p(self.a2_q), _p(self.a2_sf), _p(self.a2_deq),
             _p(self.g2), _p(self.al.offsets), _p(self.al.inv_pos), _p(self.al.plan),
             _p(tw), _p(w.prep2), _p(w.g2), _p(out), _dtype_code(out), _p(self.ws),
             self.ws.numel() * 4, s)

    def gemm1(self, variant: str, weights: Optional[ExpertWeights] = None, x=None):
        """GEMM1 alone on the layer's current buffers (for kernel timing)."""
        d, w, s = self.d, weights or self.w, _stream()
        if variant == "w4a4":
            self._gemm1_w4a4(w, s)
        else:
            call("grouped_gemm1_swiglu_w4a16", ctypes.byref(d), _p(x if x is not None else self.x_last),
                 _p(self.al.sorted_pair), _p(self.al.offsets), _p(self.al.plan), _p(w.prep13),
                 _p(w.g13), _p(self.a2_bf16), s)

    def gemm2(self, variant: str, out, weights: Optional[ExpertWeights] = None, topk_w=None):
        """GEMM2 + combine alone on the layer's current buffers (for kernel timing)."""
        d, w, s = self.d, weights or self.w, _stream()
        tw = topk_w if topk_w is not None else self.tw_last
        if variant == "w4a4":
            self._gemm2_w4a4(w, tw, out, s)
        else:
            call("grouped_gemm2_combine_w4a16", ctypes.byref(d), _p(self.a2_bf16),
                 _p(self.al.offsets), _p(self.al.inv_pos), _p(self.al.plan), _p(tw),
                 _p(w.prep2), _p(w.g2), _p(out), _dtype_code(out), _p(self.ws),
                 self.ws.numel() * 4, s)

    def forward(self, x, topk_ids, topk_w, variant: str = "w4a4", out=None,
                out_dtype=torch.bfloat16, weights: Optional[ExpertWeights] = None, marks=None):
        """Run the layer; ``marks`` = three torch.cuda.Events recorded before
        GEMM1, between the GEMMs and after GEMM2 + combine."""
        d, w = self.d, weights or self.w
        self.x_last, self.tw_last = x, topk_w
        if out is None:
            out = torch.empty(d.T, d.H, dtype=out_dtype, device=x.device)
        s = _stream()
        if variant == "w4a4":
            # Activation global scale, quantisation and the permutation (one
            # launch for decode-sized batches).
            call("moe_quantize_and_align", ctypes.byref(d), _p(x), _p(self.g1), _p(self.gs_ws),
                 self.gs_ws_bytes, _p(self.a1_q), _p(self.a1_sf), _p(self.a1_deq), _p(topk_ids),
                 _p(self.al.offsets), _p(self.al.sorted_pair), _p(self.al.inv_pos), _p(self.al.plan),
                 _p(self.al.workspace), self.al.workspace.numel(), s)
        else:
            call("moe_align", ctypes.byref(d), _p(topk_ids), _p(self.al.offsets),
                 _p(self.al.sorted_pair), _p(self.al.inv_pos), _p(self.al.plan),
                 _p(self.al.workspace), self.al.workspace.numel(), s)
        if marks:
            marks[0].record()
        if variant == "w4a4":
            g1 = lambda part, st: call(
                "grouped_gemm1_swiglu_part", ctypes.byref(d), _p(self.a1_q), _p(self.a1_sf),
                _p(self.a1_deq), _p(self.g1), _p(self.al.sorted_pair), _p(self.al.offsets),
                _p(self.al.plan), _p(w.prep13), _p(w.g13), _p(self.g2), _p(self.a2_q), _p(self.a2_sf),
                _p(self.a2_deq), part, st)
            g2 = lambda part, st: call(
                "grouped_gemm2_combine_part", ctypes.byref(d), _p(self.a2_q), _p(self.a2_sf),
                _p(self.a2_deq), _p(self.g2), _p(self.al.offsets), _p(self.al.inv_pos), _p(self.al.plan),
                _p(topk_w), _p(w.prep2), _p(w.g2), _p(out), _dtype_code(out), _p(self.ws),
                self.ws.numel() * 4, part, st)
            side = self.side if self.decoded_copies else None
        elif variant == "w4a16":
            g1 = lambda part, st: call(
                "grouped_gemm1_swiglu_w4a16_part", ctypes.byref(d), _p(x), _p(self.al.sorted_pair),
                _p(self.al.offsets), _p(self.al.plan), _p(w.prep13), _p(w.g13), _p(self.a2_bf16), part, st)
            g2 = lambda part, st: call(
                "grouped_gemm2_combine_w4a16_part", ctypes.byref(d), _p(self.a2_bf16),
                _p(self.al.offsets), _p(self.al.inv_pos), _p(self.al.plan), _p(topk_w),
                _p(w.prep2), _p(w.g2), _p(out), _dtype_code(out), _p(self.ws),
                self.ws.numel() * 4, part, st)
            side = self.side
        else:
            raise ValueError(variant)
        _run_gemms(side, g1, g2, marks)
        return out


def calibrate_g2(d: Dims, x, topk_ids, weights: ExpertWeights) -> torch.Tensor:
    """A static intermediate global scale from the GPU path itself: the
    global scale of the W4A16 intermediate (bf16 SwiGLU output) of this
    batch."""
    al = moe_align(d, topk_ids)
    a2 = gemm1_w4a16(d, x, al, weights)
    P = d.T * d.topk + d.shared * d.T
    return global_scale(a2[:P])
