"""Seeded synthetic inputs for the dispatch/combine path.

This module only draws inputs: hidden states, router logits and their top-k
selection with softmax weights (the router sits upstream of the path), and
stand-in expert outputs. It holds none of the path's arithmetic and is the
one module shared by the oracle side (tests) and the GPU side (tests, bench).

Workloads (the five configurations the path is measured and checked on):

  1 tiny      T=64,    h=128,  E=8,   R=4,  K=2   high-throughput bf16 (+LL, FP8)
  2 decode    T=128,   h=7168, E=256, R=32, K=8   low-latency FP8, cap 128
  3 prefill   T=4096,  h=7168, E=256, R=32, K=8   high-throughput bf16
  4 skew      T=8192,  h=4096, E=64,  R=8,  K=6   Zipf-biased routing, bf16
  5 fp8 big   T=16384, h=7168, E=256, R=64, K=8   FP8, 1% outlier channels x50

Recipe (numpy ``default_rng(1000 + config)``; draw order x, logits, then the
expert permutation (4) or the outlier channels (5)):
  * x ~ N(0,1) fp32, rounded to bf16 (nearest-even, via torch's cast);
    config 5 first multiplies 72 = round(0.01*h) channels, drawn without
    replacement, by 50 in fp32;
  * logits ~ N(0,1) fp32 [T,E]; config 4 adds bias[perm[i]] =
    2.0*ln(i^-1.2 / sum_j j^-1.2) for i = 1..E;
  * topk_idx = the K largest logits, in descending order, ties to the lower
    expert index (stable sort of the negated logits);
  * topk_weights = softmax over the K chosen logits, in float64, stored fp32.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    T: int
    h: int
    E: int
    R: int
    K: int
    fp8: bool
    ll: bool
    cap: int = 0
    zipf_bias: bool = False
    outlier_frac: float = 0.0

    @property
    def L(self) -> int:
        return self.E // self.R

    def describe(self) -> str:
        mode = "LL" if self.ll else "HT"
        dt = "fp8" if self.fp8 else "bf16"
        return (f"{self.name}: T={self.T} h={self.h} E={self.E} R={self.R} K={self.K} "
                f"{mode} {dt}" + (f" cap={self.cap}" if self.ll else ""))


WORKLOADS = {
    1: Workload(1, "tiny", 64, 128, 8, 4, 2, fp8=False, ll=False),
    2: Workload(2, "decode", 128, 7168, 256, 32, 8, fp8=True, ll=True, cap=128),
    3: Workload(3, "prefill", 4096, 7168, 256, 32, 8, fp8=False, ll=False),
    4: Workload(4, "skew", 8192, 4096, 64, 8, 6, fp8=False, ll=False, zipf_bias=True),
    5: Workload(5, "fp8_big", 16384, 7168, 256, 64, 8, fp8=True, ll=False,
                outlier_frac=0.01),
}


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), nearest-even, using torch's cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def topk_softmax(logits: np.ndarray, K: int) -> tuple[np.ndarray, np.ndarray]:
    """Top-K experts by logit (descending, ties to the lower index) and the
    softmax of the chosen logits (float64, stored fp32)."""
    order = np.argsort(-logits, axis=1, kind="stable")[:, :K]
    chosen = np.take_along_axis(logits, order, axis=1).astype(np.float64)
    z = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return order.astype(np.int64), w


def make_inputs(cfg: int | Workload, T: int | None = None, seed: int | None = None) -> dict:
    """Draw (x bf16 bits [T,h], topk_idx int64 [T,K], topk_w fp32 [T,K]).

    ``T`` overrides the token count (same distributions), ``seed`` the seed.
    """
    wl = WORKLOADS[cfg] if isinstance(cfg, int) else cfg
    T = wl.T if T is None else T
    rng = np.random.default_rng(1000 + wl.cid if seed is None else seed)
    xf = rng.standard_normal((T, wl.h), dtype=np.float32)
    logits = rng.standard_normal((T, wl.E), dtype=np.float32)
    if wl.zipf_bias:
        perm = rng.permutation(wl.E)
        i = np.arange(1, wl.E + 1, dtype=np.float64)
        p = i ** -1.2
        bias = np.empty(wl.E, np.float64)
        bias[perm] = 2.0 * np.log(p / p.sum())
        logits = (logits + bias.astype(np.float32)).astype(np.float32)
    if wl.outlier_frac > 0:
        n_out = int(round(wl.outlier_frac * wl.h))
        cols = rng.choice(wl.h, size=n_out, replace=False)
        xf[:, cols] *= np.float32(50.0)
    topk_idx, topk_w = topk_softmax(logits, wl.K)
    return dict(x=to_bf16_bits(xf), topk_idx=topk_idx, topk_w=topk_w,
                workload=replace(wl, T=T))


def expert_outputs(n_rows: int, h: int, seed: int, device: str = "cpu"):
    """Stand-in expert outputs: bf16 N(0,1) [n_rows, h] as a torch tensor on
    ``device`` (drawn there with a seeded torch generator)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    y = torch.randn((n_rows, h), generator=g, device=device, dtype=torch.float32)
    return y.to(torch.bfloat16)


def random_routing(T: int, K: int, E: int, seed: int, p_drop: float = 0.0) -> np.ndarray:
    """Distinct random experts per token (a uniform random K-subset in random
    order); with p_drop > 0 some entries become -1 (no route)."""
    rng = np.random.default_rng(seed)
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int64)
    if p_drop > 0:
        idx[rng.random((T, K)) < p_drop] = -1
    return idx
