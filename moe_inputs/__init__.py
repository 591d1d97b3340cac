"""Seeded synthetic inputs for the NVFP4 mixture-of-experts layer.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It draws random numbers and nothing else: it holds none of the
method's arithmetic (no quantisation, no routing, no matrix products).  Every
array is produced with ``torch`` random generators on the requested device, so
the GPU side can build multi-gigabyte weights in place; a test that compares the
two sides generates once and copies the tensors to the host for the oracle.

Workloads (shapes and value distributions):

* ``tiny``     T=16,   H=256,  I=128,  E=8,   top-2,  logits N(0,1), sigma 0.02
* ``decode``   T=64,   H=2048, I=768,  E=128, top-8,  logits N(0,1), sigma 0.02
* ``prefill``  T=4096, H=2048, I=768,  E=128, top-8,  logits N(0,1), sigma 0.02
* ``large_e``  T=256,  H=4096, I=1024, E=512 + 1 shared expert, top-10,
               Zipf(1.1)-skewed logits, sigma 0.015
* ``skew``     T=8192, H=2048, I=768,  E=128, top-8, Zipf(1.3)-skewed logits
* ``ep8_share`` T=512, H=2048, I=768, E=16, top-8 (one GPU's share of
               ``prefill`` under 8-way expert parallelism)

The expert shapes follow the 30B-A3B mixture-of-experts model the pages serve
(vLLM PR #29242, "Test Plan"), and the 512-routed + 1-shared, top-10 layout is
the 397B-A17B model of FlashInfer issue #2723 ("Model" table).

Activations are N(0,1) in FP32; except in ``tiny``, 1% of the hidden channels
(chosen without replacement) are multiplied by 20 for every token, to mimic
outlier channels.  They are then rounded to bfloat16.

Router logits are FP32.  For the skewed workloads each expert e gets a fixed
popularity rank r_e (a seeded permutation of 1..E) and logit
``-s * ln(r_e) + N(0,1)``, so that expert popularity falls off like a Zipf law
with exponent ``s``: a few experts receive thousands of rows and several
receive none.

Expert weights are FP32 N(0, sigma^2): ``w13[e]`` is [2I, H] (rows [0, I) the
gate projection, rows [I, 2I) the up projection) and ``w2[e]`` is [H, I].  Each
expert matrix has its own seed, so any single expert can be regenerated on
demand.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens
    H: int            # hidden size (GEMM1 contraction, GEMM2 output)
    I: int            # expert intermediate size (GEMM2 contraction)
    E: int            # routed experts
    topk: int         # experts per token
    shared: int       # 1 if an always-on shared expert is present
    zipf_s: float     # 0.0 -> i.i.d. N(0,1) logits; > 0 -> Zipf-skewed logits
    sigma: float      # weight standard deviation
    outlier_frac: float
    seed: int

    @property
    def n_experts(self) -> int:
        """Expert slots including the shared expert (stored last)."""
        return self.E + self.shared

    @property
    def pairs(self) -> int:
        """(token, expert) pairs, counting the shared expert's T pseudo-pairs."""
        return self.T * self.topk + self.shared * self.T

    def with_tokens(self, T: int, name: Optional[str] = None) -> "Workload":
        return dataclasses.replace(self, T=T, name=name or f"{self.name}_T{T}")

    def describe(self) -> dict:
        return {"workload": self.name, "T": self.T, "H": self.H, "I": self.I,
                "E": self.E, "topk": self.topk, "shared": self.shared,
                "routing": ("zipf(%g)" % self.zipf_s) if self.zipf_s else "normal"}


WORKLOADS = {
    "tiny": Workload("tiny", 16, 256, 128, 8, 2, 0, 0.0, 0.02, 0.0, 1000),
    "decode": Workload("decode", 64, 2048, 768, 128, 8, 0, 0.0, 0.02, 0.01, 1001),
    "prefill": Workload("prefill", 4096, 2048, 768, 128, 8, 0, 0.0, 0.02, 0.01, 1002),
    "large_e": Workload("large_e", 256, 4096, 1024, 512, 10, 1, 1.1, 0.015, 0.01, 1003),
    "skew": Workload("skew", 8192, 2048, 768, 128, 8, 0, 1.3, 0.02, 0.01, 1004),
    # One GPU's share of the prefill layer under 8-way expert parallelism:
    # 16 of the 128 experts with the 4096 pairs routed to them (about 256
    # rows each), as 512 tokens routed top-8 over 16 experts.
    "ep8_share": Workload("ep8_share", 512, 2048, 768, 16, 8, 0, 0.0, 0.02, 0.01, 1005),
}

ORDER = ["tiny", "decode", "prefill", "large_e", "skew", "ep8_share"]


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def activations(w: Workload, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    """bf16 [T, H] activations with optional outlier channels."""
    T = w.T if T is None else T
    g = _gen(device, w.seed * 7919 + 1)
    x = torch.randn(T, w.H, generator=g, device=device, dtype=torch.float32)
    n_out = int(round(w.outlier_frac * w.H))
    if n_out:
        gc = _gen("cpu", w.seed * 7919 + 2)
        ch = torch.randperm(w.H, generator=gc)[:n_out].to(device)
        x[:, ch] *= 20.0
    return x.to(torch.bfloat16)


def router_logits(w: Workload, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    """FP32 [T, E] router logits (i.i.d. normal or Zipf-skewed)."""
    T = w.T if T is None else T
    g = _gen(device, w.seed * 7919 + 3)
    noise = torch.randn(T, w.E, generator=g, device=device, dtype=torch.float32)
    if not w.zipf_s:
        return noise
    gc = _gen("cpu", w.seed * 7919 + 4)
    rank = (torch.randperm(w.E, generator=gc) + 1).to(torch.float64)
    bias = (-w.zipf_s * torch.log(rank)).to(torch.float32).to(device)
    return noise + bias[None, :]


def expert_weight(w: Workload, which: int, e: int, device="cpu") -> torch.Tensor:
    """FP32 weight of expert slot ``e`` (``e == E`` is the shared expert).

    which=13 -> [2I, H] gate/up projection; which=2 -> [H, I] down projection.
    """
    if which == 13:
        shape = (2 * w.I, w.H)
    elif which == 2:
        shape = (w.H, w.I)
    else:
        raise ValueError("which must be 13 or 2")
    g = _gen(device, (w.seed * 1_000_003 + which * 65_537 + e) * 2 + 1)
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * w.sigma


def expert_weights(w: Workload, which: int, device="cpu", experts=None) -> torch.Tensor:
    """Stacked FP32 weights [n, ...] for the listed expert slots (default: all)."""
    experts = range(w.n_experts) if experts is None else experts
    return torch.stack([expert_weight(w, which, int(e), device) for e in experts])


def bytes_of_weights(w: Workload) -> int:
    """Packed NVFP4 bytes of all expert weights (codes + block scales)."""
    per = 2 * w.I * w.H + w.H * w.I
    return w.n_experts * (per // 2 + per // 16)


def flops(w: Workload) -> float:
    """Multiply-adds x2 of both expert GEMMs over all (token, expert) pairs."""
    return 2.0 * w.pairs * (2 * w.I * w.H + w.H * w.I)


def touched_bytes(w: Workload, rows_per_expert, block: int = 16) -> float:
    """Algorithmic HBM bytes of one layer pass: weights of the experts that
    receive at least one row (4-bit codes and one scale byte per ``block``
    elements: 16 for NVFP4, 32 for MXFP4), plus bf16 x and out and the routing
    arrays."""
    per_expert = (3 * w.I * w.H) // 2 + (3 * w.I * w.H) // block
    touched = sum(1 for n in rows_per_expert if n > 0)
    return touched * per_expert + 2 * 2 * w.T * w.H + 2 * 4 * w.T * w.topk


__all__ = ["Workload", "WORKLOADS", "ORDER", "activations", "router_logits",
           "expert_weight", "expert_weights", "bytes_of_weights", "flops",
           "touched_bytes"]
