"""Fit the polynomial behind the software exp2 of the PAIR256_EXP2EMU kernel
variant: p(f) ~ 2**f on f in [0, 1], minimising the maximum RELATIVE error,
by the Remez exchange algorithm (Remez, 1934). Run it to regenerate the
constants pasted into attn_fwd_kernel.hip:

    python dense_attention_forward_amd/csrc/exp2_poly_fit.py [degree]

Method: with n+2 reference points x_i, solve
    sum_k c_k x_i**k - 2**x_i = (-1)**i * E * 2**x_i
for c_0..c_n and E, move the references to the extrema of the weighted error
(p(x) - 2**x) / 2**x, and repeat until the extrema alternate with equal
magnitude. The endpoint f = 0 is pinned afterwards to c_0 = 1 exactly (so
that 2**n is exact for integer arguments) at the cost of a slightly larger
error, which the report below includes.
"""
from __future__ import annotations

import sys

import numpy as np


def remez(degree: int, iters: int = 30):
    n = degree
    x = 0.5 - 0.5 * np.cos(np.pi * np.arange(n + 2) / (n + 1))  # Chebyshev nodes on [0, 1]
    grid = np.linspace(0.0, 1.0, 200001)
    for _ in range(iters):
        A = np.zeros((n + 2, n + 2))
        for i, xi in enumerate(x):
            A[i, :n + 1] = xi ** np.arange(n + 1)
            A[i, n + 1] = -((-1.0) ** i) * 2.0 ** xi
        sol = np.linalg.solve(A, 2.0 ** x)
        c = sol[:n + 1]
        err = (np.polyval(c[::-1], grid) - 2.0 ** grid) / 2.0 ** grid
        # new references: one extremum per sign-alternating segment
        sign_change = np.where(np.diff(np.sign(err)) != 0)[0]
        bounds = np.concatenate(([0], sign_change + 1, [len(grid)]))
        ext = [b0 + int(np.argmax(np.abs(err[b0:b1]))) for b0, b1 in zip(bounds[:-1], bounds[1:])]
        if len(ext) != n + 2:
            break
        x = grid[ext]
    return c


def pinned(c):
    """Force c_0 = 1 and refit c_1..c_n (least max error by a final Remez-free
    least-squares polish on the relative error)."""
    grid = np.linspace(0.0, 1.0, 20001)
    n = len(c) - 1
    A = np.stack([grid ** k for k in range(1, n + 1)], axis=1) / (2.0 ** grid)[:, None]
    b = 1.0 - 1.0 / 2.0 ** grid
    # minimise the max of |A c' - b| by iteratively reweighted least squares
    w = np.ones_like(grid)
    for _ in range(200):
        cw, *_ = np.linalg.lstsq(A * w[:, None], b * w, rcond=None)
        r = np.abs(A @ cw - b)
        w = w * (r / r.max() + 1e-3) ** 0.5
    return np.concatenate(([1.0], cw))


def report(c):
    f = np.linspace(0.0, 1.0, 1000001)
    rel = (np.polyval(np.asarray(c, dtype=np.float32).astype(np.float64)[::-1], f) - 2.0 ** f) / 2.0 ** f
    return np.abs(rel).max()


if __name__ == "__main__":
    deg = int(sys.argv[1]) if len(sys.argv) > 1 else 3
    c = pinned(remez(deg))
    c32 = [float(np.float32(v)) for v in c]
    print(f"// degree {deg}, max relative error on [0, 1] with float32 coefficients: {report(c32):.3e}")
    for k, v in enumerate(c32):
        print(f"constexpr float kExp2C{k} = {v!r}f;")
