"""Seeded synthetic inputs for the dense attention forward workloads.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests, and therefore holds no attention arithmetic: only shapes, seeds,
value distributions and the bf16 cast of the drawn numbers.

Workloads (all bf16, head_dim 128, tensors laid out [B, H, S, D]):

  name            B   H      S  Q / K                     V
  s256            1   1    256  N(0,1)                    N(0,1)
  s1k             2  16   1024  N(0,1)                    N(0,1)
  s4k             4  16   4096  N(0,1)                    N(0,1)
  s8k_peaked      2  16   8192  N(0, std 2)               U(-1,1)
  s16k_outliers   1  16  16384  N(0,1); 1% of K rows x8   N(0,1)

The 4K/8K/16K sequence lengths stand in for the benchmark shapes the
B200 attention-kernel article ("B200 attention kernel from scratch to
~SOTA in 60 figures", "About this blog") measures on; its batch and head
counts are not printed there, so B*S = 16384 tokens and H = 16 are used.

Recipe: a CPU ``torch.Generator`` seeded with 1000 + the workload's index
(1..5) draws Q, then K, then V in float32; each is cast to bf16 with
round-to-nearest-even. For the outlier workload, after V is drawn, each
(b, h) in order takes ``randperm(S)[:round(0.01*S)]`` from the same
generator and those K rows are multiplied by 8 (exact in bf16).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Tuple

import torch

HEAD_DIM = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int            # 1-based position in the workload list
    B: int
    H: int
    S: int
    D: int
    qk_dist: str          # "normal" (std qk_std) for Q and K
    qk_std: float
    v_dist: str           # "normal" or "uniform"
    outlier_frac: float   # fraction of K rows per (b, h) multiplied by outlier_mult
    outlier_mult: float
    scale: float          # softmax scale handed to the kernel, as a float32 value

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def flops(self) -> int:
        """Flops of the two matrix products (QK^T and PV): 4*B*H*S*S*D."""
        return 4 * self.B * self.H * self.S * self.S * self.D

    @property
    def shape(self) -> Tuple[int, int, int, int]:
        return (self.B, self.H, self.S, self.D)

    def describe(self) -> str:
        return (f"{self.name}: B={self.B} H={self.H} S={self.S} D={self.D} "
                f"QK~{self.qk_dist}(std {self.qk_std}) V~{self.v_dist} "
                f"outliers={self.outlier_frac} x{self.outlier_mult} seed={self.seed}")


def _f32(x: float) -> float:
    return float(torch.tensor(x, dtype=torch.float32).item())


# 1/sqrt(128) rounded to float32: the scale value the kernel receives.
DEFAULT_SCALE = _f32(1.0 / math.sqrt(HEAD_DIM))

WORKLOADS = [
    Workload("s256", 1, 1, 1, 256, 128, "normal", 1.0, "normal", 0.0, 1.0, DEFAULT_SCALE),
    Workload("s1k", 2, 2, 16, 1024, 128, "normal", 1.0, "normal", 0.0, 1.0, DEFAULT_SCALE),
    Workload("s4k", 3, 4, 16, 4096, 128, "normal", 1.0, "normal", 0.0, 1.0, DEFAULT_SCALE),
    Workload("s8k_peaked", 4, 2, 16, 8192, 128, "normal", 2.0, "uniform", 0.0, 1.0, DEFAULT_SCALE),
    Workload("s16k_outliers", 5, 1, 16, 16384, 128, "normal", 1.0, "normal", 0.01, 8.0, DEFAULT_SCALE),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def get(name: str) -> Workload:
    return BY_NAME[name]


def _draw(gen: torch.Generator, shape, dist: str, std: float) -> torch.Tensor:
    if dist == "normal":
        t = torch.randn(shape, generator=gen, dtype=torch.float32)
        if std != 1.0:
            t = t * std
        return t
    if dist == "uniform":
        return torch.rand(shape, generator=gen, dtype=torch.float32) * 2.0 - 1.0
    raise ValueError(dist)


def outlier_rows(S: int, frac: float) -> int:
    return int(round(frac * S))


def make_inputs(w: Workload, B: int | None = None, H: int | None = None, S: int | None = None):
    """Draw (q, k, v) as contiguous bf16 CPU tensors of shape [B, H, S, D].

    B/H/S may be overridden to draw a smaller tensor with the same recipe
    (used for parity cases that the oracle must finish in seconds)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    S = w.S if S is None else S
    shape = (B, H, S, w.D)
    gen = torch.Generator().manual_seed(w.seed)
    q = _draw(gen, shape, w.qk_dist, w.qk_std)
    k = _draw(gen, shape, w.qk_dist, w.qk_std)
    v = _draw(gen, shape, w.v_dist, 1.0)
    if w.outlier_frac > 0:
        n = outlier_rows(S, w.outlier_frac)
        for b in range(B):
            for h in range(H):
                rows = torch.randperm(S, generator=gen)[:n]
                k[b, h, rows] *= w.outlier_mult
    return (q.to(torch.bfloat16).contiguous(), k.to(torch.bfloat16).contiguous(),
            v.to(torch.bfloat16).contiguous())


def make_random(B: int, H: int, S: int, D: int, seed: int, qk_std: float = 1.0,
                v_dist: str = "normal", outlier_frac: float = 0.0, outlier_mult: float = 8.0):
    """Same recipe as ``make_inputs`` for an arbitrary shape and seed."""
    w = Workload("adhoc", seed - 1000, B, H, S, D, "normal", qk_std, v_dist,
                 outlier_frac, outlier_mult, DEFAULT_SCALE)
    return make_inputs(w)


def staircase_keys(k: torch.Tensor, tile: int = 128, step: float = 20.0) -> torch.Tensor:
    """K with its rows in key tile t (of `tile` keys) multiplied by
    0.25 + step * t, cast back to bf16: each tile's largest scores rise well
    above the previous tile's, so an online softmax moves its base on nearly
    every tile (a test pattern for the lazy rescale)."""
    S = k.shape[2]
    f = 0.25 + step * (torch.arange(S) // tile).to(torch.float32)
    return (k.float() * f.reshape(1, 1, S, 1)).to(torch.bfloat16).contiguous()


def dominant_key_small_lse_case():
    """One query e_0 over 256 keys whose first components are -45.25 (key 0),
    10.375 (key 200) and -340 (all others): key 200 carries nearly all the
    weight, lands 7.1 base-2 units above the first tile's max (below the
    rebase threshold, so its p = 2^7.1 is not exact in bf16), and lse is
    close to 0.92, where the relative LSE bar is an absolute one. Every value
    is exact in bf16."""
    S = 256
    q = torch.zeros((1, 1, 1, 128))
    q[0, 0, 0, 0] = 1.0
    k = torch.zeros((1, 1, S, 128))
    k[0, 0, :, 0] = -340.0
    k[0, 0, 0, 0] = -45.25
    k[0, 0, 200, 0] = 10.375
    v = torch.zeros((1, 1, S, 128))
    v[0, 0, :, 1] = torch.linspace(-1.0, 1.0, S)
    v[0, 0, 200, 2] = 1.0
    return tuple(t.to(torch.bfloat16) for t in (q, k, v))
