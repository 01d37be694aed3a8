"""Seeded synthetic inputs for the per-expert mixed-precision MoE layer.

This module only draws random numbers and describes workload shapes. It holds
none of the method's arithmetic (no quantizer, router, allocator or FFN), so
both the CPU oracle and the GPU library can be fed from it without sharing any
computation.

Workloads (all SwiGLU experts; W1 = gate, W3 = up, W2 = down):

* ``tiny``           E=8,   d=256,  F=512,   top-2, 16 tokens, fixed bits
* ``decode_coarse``  E=8,   d=4096, F=14336, top-2, 1/4/16 tokens, avg 4.5 bits
* ``decode_fine``    E=128, d=2048, F=768,   top-8, 64 tokens, avg 4 bits,
                     0.1% weight outliers x20
* ``prefill``        E=64,  d=4096, F=1408,  top-6, 4096 tokens, avg 5 bits
* ``dynamic``        the decode_fine layer with fp16 masters and a budget
                     stepped through avg 8, 6, 4, 3.5, 5 bits every 8 steps

``kv_trace`` draws a KV-cache occupancy trace (sequences arriving, growing
and finishing) for the budget scheduler.

Distributions: weights N(0, 0.02) in fp32 (optionally with Bernoulli outliers
multiplied by 20, optionally rounded to fp16), router logits N(0, 1) in fp32,
activations N(0, 1) rounded to bf16 (round to nearest even), expert
importance p_e proportional to (e+1)^(-s) (Zipf) and normalised.

Every tensor comes from its own ``torch.Generator`` whose seed is derived from
(seed, workload name, tensor name, step), so a tensor is reproducible on its
own. Generation on ``cuda`` and on ``cpu`` use different generators and give
different values: a test draws on one device and copies to the other.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional, Sequence

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    E: int
    d: int
    F: int
    k: int
    T: int
    bits: Optional[Sequence[int]] = None      # fixed bit-widths (tiny)
    budget_avg: Optional[float] = None        # budget as average bits/weight
    zipf_s: Optional[float] = None            # importance exponent
    outlier_rate: float = 0.0
    outlier_mult: float = 20.0
    master: str = "f32"                       # "f32" or "f16"
    w_std: float = 0.02
    schedule: Optional[Sequence[float]] = None  # dynamic: avg bits per phase
    steps_per_phase: int = 0
    renorm: int = 0

    @property
    def W_e(self) -> int:
        """Weight elements per expert: W1, W3 (F x d) and W2 (d x F)."""
        return 3 * self.d * self.F

    def budget_bits(self, avg: Optional[float] = None) -> int:
        a = self.budget_avg if avg is None else avg
        # avg may be fractional (3.5, 4.5): the product is an integer for
        # every workload here because W_e is even.
        return int(round(a * 2)) * self.E * self.W_e // 2

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", E=8, d=256, F=512, k=2, T=16,
                     bits=(8, 4, 4, 3, 3, 3, 8, 4)),
    "decode_coarse": Workload("decode_coarse", E=8, d=4096, F=14336, k=2, T=16,
                              budget_avg=4.5, zipf_s=1.0),
    "decode_fine": Workload("decode_fine", E=128, d=2048, F=768, k=8, T=64,
                            budget_avg=4.0, zipf_s=1.1, outlier_rate=0.001),
    "prefill": Workload("prefill", E=64, d=4096, F=1408, k=6, T=4096,
                        budget_avg=5.0, zipf_s=1.0),
    "dynamic": Workload("dynamic", E=128, d=2048, F=768, k=8, T=64,
                        budget_avg=8.0, zipf_s=1.1, outlier_rate=0.001,
                        master="f16", schedule=(8, 6, 4, 3.5, 5),
                        steps_per_phase=8),
}

DECODE_COARSE_BATCHES = (1, 4, 16)


def _seed(*parts) -> int:
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def zipf_importance(E: int, s: float):
    """p_e proportional to (e+1)^(-s), normalised; rank = expert index."""
    import numpy as np
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-float(s))
    return p / p.sum()


def expert_weights(wl: Workload, device="cpu", seed: int = 0):
    """Return (w1 [E,F,d], w3 [E,F,d], w2 [E,d,F]) masters.

    fp32 N(0, w_std); with outliers a Bernoulli(rate) mask multiplies
    weights by outlier_mult; fp16 masters are the fp32 draw rounded to fp16.
    """
    out = []
    for name, shape in (("w1", (wl.E, wl.F, wl.d)), ("w3", (wl.E, wl.F, wl.d)),
                        ("w2", (wl.E, wl.d, wl.F))):
        g = _gen(device, seed, wl.name, wl.E, wl.d, wl.F, name)
        w = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        w.mul_(wl.w_std)
        if wl.outlier_rate > 0:
            g2 = _gen(device, seed, wl.name, wl.E, wl.d, wl.F, name, "outliers")
            mask = torch.rand(shape, generator=g2, device=device) < wl.outlier_rate
            w = torch.where(mask, w * wl.outlier_mult, w)
        if wl.master == "f16":
            w = w.to(torch.float16)
        out.append(w.contiguous())
    return tuple(out)


def tokens(wl: Workload, T: Optional[int] = None, device="cpu", seed: int = 0,
           step: int = 0):
    """Return (x bf16 [T,d], logits fp32 [T,E]) for one batch."""
    T = wl.T if T is None else T
    gx = _gen(device, seed, wl.name, wl.E, wl.d, "x", T, step)
    gl = _gen(device, seed, wl.name, wl.E, wl.d, "logits", T, step)
    x = torch.randn((T, wl.d), generator=gx, device=device, dtype=torch.float32)
    x = x.to(torch.bfloat16)   # round to nearest even
    logits = torch.randn((T, wl.E), generator=gl, device=device, dtype=torch.float32)
    return x.contiguous(), logits.contiguous()


def importance(wl: Workload):
    if wl.zipf_s is None:
        import numpy as np
        return np.full(wl.E, 1.0 / wl.E)
    return zipf_importance(wl.E, wl.zipf_s)


def kv_trace(steps: int, kv_peak_bytes: int, seed: int = 0, name: str = "kv"):
    """KV-cache occupancy in bytes over ``steps`` decode steps: sequences
    arrive (probability 0.35 per step, with a prompt of 1..64 tokens), grow by
    one token per step and finish (probability 0.04 per step); a token takes
    kv_peak_bytes / 1024 bytes. Occupancy is capped at kv_peak_bytes."""
    import random
    rng = random.Random(_seed(seed, name, steps, kv_peak_bytes))
    per_token = max(1, kv_peak_bytes // 1024)
    live, out = [], []
    for _ in range(steps):
        if rng.random() < 0.35:
            live.append(rng.randrange(1, 65))
        out.append(min(kv_peak_bytes, sum(live) * per_token))
        live = [t + 1 for t in live if rng.random() >= 0.04]
    return out
