"""Tile-by-tile fp64 model of the article's online-softmax algorithm.

TEST INFRASTRUCTURE ONLY (same rule as the two-pass oracle: tests, the
smoke check and the benchmark's CPU-baseline leg only).

It walks the K/V sequence one tile at a time for each 128-row query tile,
in the order of "B200 attention kernel from scratch to ~SOTA in 60
figures":

* Chapter 1, section B (online softmax update): take the tile's row max,
  move to a new base, rescale the running row sum and the O accumulator
  by the ratio of the old and new base, form unnormalised P against the
  base, add its row sums, accumulate P.V; after the last tile divide O by
  the row sum. The first tile has no earlier state, so it sets the base
  and the sums directly (no rescale pass).
* Chapter 8 (hardware approximations): exponentials are base 2 with
  scale*log2(e) folded into the score scale; the max is taken over raw
  scores and multiplied by that factor afterwards (valid for a positive
  scale); results below 2^-126 flush to zero instead of being kept as
  subnormals.
* Chapter 11 (skip O rescale): keep the current base unless the new
  tile's scaled max exceeds it by at least REBASE_THRESH_LOG2 = 8 (base-2
  units); only then rebase and rescale. The per-row decision is modelled
  per row, which is what a warp-wide "any row" pass computes for every
  row (rows that did not rebase get a factor of 1).

With ``p_to_bf16=False`` every step is exact in real arithmetic, so the
result must equal the two-pass oracle up to fp64 rounding: that is the
article's claim that skipping a rescale loses no information. With
``p_to_bf16=True`` P is rounded to bf16 (round to nearest even) before the
P.V product while the row sum keeps the unrounded P (Chapter 1, section B,
P written as bf16 after adding to the row sum); that variant estimates the
error a kernel with bf16 P has, it is not the reference result.
``rowsum_of_rounded=True`` (with ``p_to_bf16``) instead sums the same
rounded P that enters P.V, so O is divided by exactly the total weight its
accumulator received and stays a convex combination of V rows. Where a
few large P dominate a row and round the same way, the unrounded sum
leaves a bias of up to 2^-9 relative on the whole row; summing the rounded
values removes it.
"""
from __future__ import annotations

import math
from typing import Tuple

import torch

LOG2E = 1.0 / math.log(2.0)
REBASE_THRESH_LOG2 = 8.0
FTZ_LIMIT = 2.0 ** -126


def natural_gap(log2_gap: float) -> float:
    """A gap in base-2 exponent units expressed in natural-exponent units."""
    return log2_gap / LOG2E


def raw_score_gap(log2_gap: float, head_dim: int) -> float:
    """A base-2 gap expressed in raw q.k units when scale = 1/sqrt(head_dim)."""
    return natural_gap(log2_gap) * math.sqrt(head_dim)


def unnormalised_peak(log2_gap: float) -> float:
    """Largest unnormalised P when a tile's max exceeds the kept base by log2_gap."""
    return 2.0 ** log2_gap


def _ftz(x: torch.Tensor) -> torch.Tensor:
    return torch.where(x.abs() < FTZ_LIMIT, torch.zeros_like(x), x)


def _bf16_rne(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def online_tile(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sigma: float,
                block_n: int, thresh_log2: float = REBASE_THRESH_LOG2,
                p_to_bf16: bool = False, stats: dict | None = None,
                rowsum_of_rounded: bool = False):
    """One query tile q [M, D] against k, v [S, D] (float64). Returns (O [M, D], lse [M])."""
    M = q.shape[0]
    S = k.shape[0]
    c = sigma * LOG2E                                   # folded scale, base-2 units
    kept = torch.zeros(M, dtype=torch.float64)          # base in base-2 units
    rowsum = torch.zeros(M, dtype=torch.float64)
    acc = torch.zeros((M, v.shape[1]), dtype=torch.float64)
    rebases = 0
    row_rebases = torch.zeros(M, dtype=torch.int64)    # rebases after the first tile, per row
    for j0 in range(0, S, block_n):
        kt = k[j0:j0 + block_n]
        vt = v[j0:j0 + block_n]
        s_raw = q @ kt.transpose(0, 1)                  # raw scores, no scale
        tile_max = s_raw.max(dim=1).values * c          # max of raw scores, then scaled
        if j0 == 0:
            kept = tile_max.clone()                     # first tile sets the base
        else:
            cand = torch.maximum(kept, tile_max)
            need = (cand - kept) >= thresh_log2
            alpha = torch.where(need, _ftz(torch.exp2(kept - cand)), torch.ones_like(kept))
            rowsum = rowsum * alpha
            acc = acc * alpha[:, None]
            kept = torch.where(need, cand, kept)
            rebases += int(need.sum())
            row_rebases += need.to(torch.int64)
        p = _ftz(torch.exp2(s_raw * c - kept[:, None]))  # unnormalised P against the kept base
        if stats is not None:
            stats["max_p"] = max(stats.get("max_p", 0.0), float(p.max()))
        pv = _bf16_rne(p) if p_to_bf16 else p
        rowsum = rowsum + (pv if rowsum_of_rounded else p).sum(dim=1)
        acc = acc + pv @ vt
    if stats is not None:
        stats["rebases"] = stats.get("rebases", 0) + rebases
        stats.setdefault("row_rebases", []).append(row_rebases)
    o = acc / rowsum[:, None]
    lse = (kept + torch.log2(rowsum)) * math.log(2.0)   # natural log of the denominator
    return o, lse


def online_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float,
                     block_m: int = 128, block_n: int = 128,
                     thresh_log2: float = REBASE_THRESH_LOG2, p_to_bf16: bool = False,
                     stats: dict | None = None,
                     rowsum_of_rounded: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Online-softmax attention over [B, H, S, D] inputs; returns float64 (O, lse)."""
    if scale <= 0:
        raise ValueError("the max of raw scores commutes with the scale only for scale > 0")
    sigma = float(torch.tensor(scale, dtype=torch.float32).item())
    B, H, S, D = q.shape
    o = torch.empty((B, H, S, v.shape[3]), dtype=torch.float64)
    lse = torch.empty((B, H, S), dtype=torch.float64)
    for b in range(B):
        for h in range(H):
            kd = k[b, h].to(torch.float64)
            vd = v[b, h].to(torch.float64)
            for i0 in range(0, S, block_m):
                qd = q[b, h, i0:i0 + block_m].to(torch.float64)
                o[b, h, i0:i0 + block_m], lse[b, h, i0:i0 + block_m] = online_tile(
                    qd, kd, vd, sigma, block_n, thresh_log2, p_to_bf16, stats, rowsum_of_rounded)
    return o, lse
