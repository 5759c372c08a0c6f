"""CPU fp64 oracle for the dense attention forward.

TEST INFRASTRUCTURE ONLY. Only tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the GPU product path never does.

What it computes is the plain definition of softmax attention (the
"B200 attention kernel from scratch to ~SOTA in 60 figures" article,
Chapter 1 "ii. Work parallelization" and section B, "online softmax"):
for every batch b, head h and query row i, with q, k, v the bf16 inputs
widened exactly to float64 and sigma = float64(float32(scale)),

    s_ij  = sigma * sum_d q_id k_jd
    m_i   = max_j s_ij
    l_i   = sum_j exp(s_ij - m_i)
    O_i   = (sum_j exp(s_ij - m_i) v_j) / l_i
    lse_i = m_i + ln(l_i)                      (natural log)

The article's method reaches exactly this result (up to rounding order):
its online update rescales running sums by exact factors, so the two-pass
definition above is the oracle. Nothing is rounded back to bf16 or fp32.
The work is blocked over query rows only so a block's score matrix fits
in memory; every row still sees all keys at once. The log-sum-exp output
is not defined in the article; it is read as the natural log of the full
softmax denominator including the scale.

Pinned by tests against closed forms, invariants, brute force on tiny
inputs and torch's scaled_dot_product_attention in fp64 (see the
oracle's test module).
"""
from __future__ import annotations

from typing import Iterable, Tuple

import torch

__all__ = ["attention", "attention_rows", "attention_probs", "sigma_of"]


def sigma_of(scale: float) -> float:
    """The scale as the GPU receives it: rounded to float32, widened to float64."""
    return float(torch.tensor(scale, dtype=torch.float32).item())


def _head(qd: torch.Tensor, kd: torch.Tensor, vd: torch.Tensor, sigma: float):
    """Two-pass softmax attention for one head's query rows qd [R, D] against kd, vd [S, D]."""
    s = (qd @ kd.transpose(0, 1)) * sigma          # [R, S] scores
    m = s.max(dim=1, keepdim=True).values          # pass 1: row max
    e = torch.exp(s - m)                           # pass 2: shifted exponentials
    l = e.sum(dim=1, keepdim=True)                 # row sums
    o = (e @ vd) / l                               # normalised weighted sum of values
    lse = m.squeeze(1) + torch.log(l.squeeze(1))
    return o, lse


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float,
              block_rows: int = 1024) -> Tuple[torch.Tensor, torch.Tensor]:
    """Return (O, lse) in float64 for [B, H, S, D] inputs (any float dtype, CPU)."""
    if (q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or q.shape[:2] != k.shape[:2]
            or v.shape[:3] != k.shape[:3] or q.shape[3] != k.shape[3]):
        raise ValueError(f"bad shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    B, H, S_q, D = q.shape
    sigma = sigma_of(scale)
    o = torch.empty((B, H, S_q, v.shape[3]), dtype=torch.float64)
    lse = torch.empty((B, H, S_q), dtype=torch.float64)
    for b in range(B):
        for h in range(H):
            kd = k[b, h].to(torch.float64)
            vd = v[b, h].to(torch.float64)
            for r0 in range(0, S_q, block_rows):
                r1 = min(S_q, r0 + block_rows)
                qd = q[b, h, r0:r1].to(torch.float64)
                o[b, h, r0:r1], lse[b, h, r0:r1] = _head(qd, kd, vd, sigma)
    return o, lse


def attention_rows(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float,
                   picks: Iterable[Tuple[int, int, int]]) -> Tuple[torch.Tensor, torch.Tensor]:
    """(O, lse) in float64 for selected (b, h, row) triples only: [n, D] and [n]."""
    sigma = sigma_of(scale)
    picks = list(picks)
    o = torch.empty((len(picks), v.shape[3]), dtype=torch.float64)
    lse = torch.empty((len(picks),), dtype=torch.float64)
    by_head = {}
    for n, (b, h, i) in enumerate(picks):
        by_head.setdefault((b, h), []).append((n, i))
    for (b, h), items in by_head.items():
        idx = torch.tensor([i for _, i in items])
        out_idx = torch.tensor([n for n, _ in items])
        oo, ll = _head(q[b, h, idx].to(torch.float64), k[b, h].to(torch.float64),
                       v[b, h].to(torch.float64), sigma)
        o[out_idx] = oo
        lse[out_idx] = ll
    return o, lse


def attention_probs(q: torch.Tensor, k: torch.Tensor, scale: float) -> torch.Tensor:
    """The full softmax matrix P [B, H, S_q, S_k] in float64 (small inputs only)."""
    sigma = sigma_of(scale)
    s = (q.to(torch.float64) @ k.to(torch.float64).transpose(-1, -2)) * sigma
    m = s.max(dim=-1, keepdim=True).values
    e = torch.exp(s - m)
    return e / e.sum(dim=-1, keepdim=True)
