"""Pins of the CPU oracle: checks that do not reuse the oracle's own formula.

Each pin takes an ``attn(q, k, v, scale) -> (o, lse)`` callable with the
oracle's contract (float64 results, the scale rounded to float32 first) and
raises AssertionError on a mismatch. They run against the oracle itself
(must pass) and against copies of it with one planted mistake (each such
mutant must fail at least one pin).

What fixes each expected value:
  * two_keys, orthogonal_keys, single_key: closed forms of a softmax over
    two or four distinct scores, written with sigmoid/softplus-style
    formulas instead of max/exp/sum;
  * q_zero, identical_keys: all scores equal, so O is the mean of V and the
    log-sum-exp is the common score plus ln(S);
  * key_shift, permutation, affine_v, dominant_key: invariants of the
    definition (a shift added to every score, reordering, linearity of the
    weighted mean, a saturated softmax);
  * brute_force: scalar Python loops over a tiny case;
  * sdpa: torch's scaled_dot_product_attention and logsumexp in float64;
  * inexact_scale: the two-key closed form with a scale (0.1) that float32
    cannot hold exactly, at scores large enough that using the unrounded
    scale moves O and lse far beyond the tolerance.

Pins of the probability matrix take ``probs(q, k, scale) -> P`` instead
(PROB_PINS): the two-key sigmoid closed form, the orthogonal-key closed
form, and P.V against the brute-force weighted mean.
"""
from __future__ import annotations

import math
import struct

import torch

F64 = torch.float64
SCALE = 0.5  # exactly representable in float32, so sigma == SCALE


def _t(x):
    return torch.tensor(x, dtype=F64)


def _close(a, b, tol, what):
    a = torch.as_tensor(a, dtype=F64)
    b = torch.as_tensor(b, dtype=F64)
    if a.shape != b.shape:
        raise AssertionError(f"{what}: shape {tuple(a.shape)} != {tuple(b.shape)}")
    if not torch.isfinite(a).all():
        raise AssertionError(f"{what}: non-finite values")
    err = (a - b).abs().max().item() if a.numel() else 0.0
    if not err <= tol:
        raise AssertionError(f"{what}: max error {err:.3e} > {tol:.1e}")


def pin_two_keys(attn):
    """One query (D=1, q=1) and keys 0 and a: the weight of key 1 is
    sigmoid(sigma*a) and lse = softplus(sigma*a); includes sigma*a = 1000,
    where exp without subtracting the max overflows."""
    for a in (0.0, 1.0, -3.0, 40.0, 2000.0):
        v0, v1 = 0.25, -1.5
        q = _t([[[[1.0]]]])
        k = _t([[[[0.0], [a]]]])
        v = _t([[[[v0], [v1]]]])
        o, lse = attn(q, k, v, SCALE)
        x = SCALE * a
        w1 = 1.0 / (1.0 + math.exp(-x)) if x >= 0 else math.exp(x) / (1.0 + math.exp(x))
        _close(o, _t([[[[v0 + (v1 - v0) * w1]]]]), 1e-13, f"two_keys O a={a}")
        soft = max(x, 0.0) + math.log1p(math.exp(-abs(x)))
        _close(lse, _t([[[soft]]]), 1e-12, f"two_keys lse a={a}")


def pin_orthogonal_keys(attn):
    """K = c*I (4 keys, D=4), query i = unit vector pi(i) with pi a 4-cycle:
    query i weighs key pi(i) by e^(sigma c) and the other three by 1.
    V has 3 columns, so a transposed operand cannot go unnoticed."""
    c = 3.0
    pi = [1, 2, 3, 0]
    q = torch.zeros((1, 1, 4, 4), dtype=F64)
    for i, j in enumerate(pi):
        q[0, 0, i, j] = 1.0
    k = (c * torch.eye(4, dtype=F64)).reshape(1, 1, 4, 4)
    gen = torch.Generator().manual_seed(7)
    v = torch.randn((1, 1, 4, 3), generator=gen, dtype=F64)
    o, lse = attn(q, k, v, SCALE)
    big = math.exp(SCALE * c)
    exp_o = torch.empty((4, 3), dtype=F64)
    for i in range(4):
        tot = v[0, 0].sum(dim=0) - v[0, 0, pi[i]]
        exp_o[i] = (big * v[0, 0, pi[i]] + tot) / (big + 3.0)
    _close(o[0, 0], exp_o, 1e-13, "orthogonal_keys O")
    _close(lse[0, 0], torch.full((4,), math.log(big + 3.0), dtype=F64), 1e-13, "orthogonal_keys lse")


def pin_q_zero(attn):
    """Q = 0: every score is 0, so O is the column mean of V and lse = ln S."""
    gen = torch.Generator().manual_seed(11)
    S = 7
    q = torch.zeros((2, 1, 5, 6), dtype=F64)
    k = torch.randn((2, 1, S, 6), generator=gen, dtype=F64)
    v = torch.randn((2, 1, S, 3), generator=gen, dtype=F64)
    o, lse = attn(q, k, v, SCALE)
    _close(o, v.mean(dim=2, keepdim=True).expand(2, 1, 5, 3), 1e-14, "q_zero O")
    _close(lse, torch.full((2, 1, 5), math.log(S), dtype=F64), 1e-14, "q_zero lse")


def pin_identical_keys(attn):
    """All keys equal k0: O is the column mean of V, lse = sigma q.k0 + ln S."""
    gen = torch.Generator().manual_seed(12)
    S = 9
    q = torch.randn((1, 2, 4, 5), generator=gen, dtype=F64)
    k0 = torch.randn((5,), generator=gen, dtype=F64)
    k = k0.expand(1, 2, S, 5).clone()
    v = torch.randn((1, 2, S, 2), generator=gen, dtype=F64)
    o, lse = attn(q, k, v, SCALE)
    _close(o, v.mean(dim=2, keepdim=True).expand(1, 2, 4, 2), 1e-13, "identical_keys O")
    exp_lse = torch.empty((1, 2, 4), dtype=F64)
    for h in range(2):
        for i in range(4):
            exp_lse[0, h, i] = SCALE * float(sum(q[0, h, i, d] * k0[d] for d in range(5))) + math.log(S)
    _close(lse, exp_lse, 1e-13, "identical_keys lse")


def pin_key_shift(attn):
    """Adding u to every key adds sigma q_i.u to every score of row i: O is
    unchanged and lse_i moves by sigma q_i.u."""
    gen = torch.Generator().manual_seed(13)
    q = torch.randn((1, 1, 6, 4), generator=gen, dtype=F64)
    k = torch.randn((1, 1, 10, 4), generator=gen, dtype=F64)
    v = torch.randn((1, 1, 10, 3), generator=gen, dtype=F64)
    u = torch.tensor([0.5, -2.0, 1.25, 3.0], dtype=F64)
    o1, lse1 = attn(q, k, v, SCALE)
    o2, lse2 = attn(q, k + u, v, SCALE)
    _close(o2, o1, 1e-12, "key_shift O")
    shift = torch.tensor([SCALE * sum(float(q[0, 0, i, d]) * float(u[d]) for d in range(4))
                          for i in range(6)], dtype=F64)
    _close(lse2[0, 0] - lse1[0, 0], shift, 1e-12, "key_shift lse")


def pin_permutation(attn):
    """Reordering keys and values together changes nothing; reordering the
    queries reorders O and lse the same way."""
    gen = torch.Generator().manual_seed(14)
    q = torch.randn((1, 1, 5, 4), generator=gen, dtype=F64)
    k = torch.randn((1, 1, 8, 4), generator=gen, dtype=F64)
    v = torch.randn((1, 1, 8, 3), generator=gen, dtype=F64)
    o, lse = attn(q, k, v, SCALE)
    pk = torch.tensor([3, 0, 7, 1, 6, 2, 5, 4])
    o2, lse2 = attn(q, k[:, :, pk], v[:, :, pk], SCALE)
    _close(o2, o, 1e-13, "permutation(keys) O")
    _close(lse2, lse, 1e-13, "permutation(keys) lse")
    pq = torch.tensor([4, 2, 0, 1, 3])
    o3, lse3 = attn(q[:, :, pq], k, v, SCALE)
    _close(o3, o[:, :, pq], 1e-13, "permutation(queries) O")
    _close(lse3, lse[:, :, pq], 1e-13, "permutation(queries) lse")


def pin_affine_v(attn):
    """O is a convex combination of V's rows: V A + 1 b^T gives O A + 1 b^T."""
    gen = torch.Generator().manual_seed(15)
    q = torch.randn((1, 1, 5, 4), generator=gen, dtype=F64)
    k = torch.randn((1, 1, 6, 4), generator=gen, dtype=F64)
    v = torch.randn((1, 1, 6, 3), generator=gen, dtype=F64)
    A = torch.randn((3, 2), generator=gen, dtype=F64)
    bvec = torch.tensor([1.5, -0.5], dtype=F64)
    o, _ = attn(q, k, v, SCALE)
    o2, _ = attn(q, k, v @ A + bvec, SCALE)
    _close(o2, o @ A + bvec, 1e-12, "affine_v O")


def pin_single_key(attn):
    """One key: its value is the output and lse is its scaled score."""
    gen = torch.Generator().manual_seed(16)
    q = torch.randn((1, 1, 3, 4), generator=gen, dtype=F64)
    k = torch.randn((1, 1, 1, 4), generator=gen, dtype=F64)
    v = torch.randn((1, 1, 1, 5), generator=gen, dtype=F64)
    o, lse = attn(q, k, v, SCALE)
    _close(o, v.expand(1, 1, 3, 5), 1e-14, "single_key O")
    exp_lse = torch.tensor([SCALE * sum(float(q[0, 0, i, d]) * float(k[0, 0, 0, d]) for d in range(4))
                            for i in range(3)], dtype=F64)
    _close(lse[0, 0], exp_lse, 1e-13, "single_key lse")


def pin_dominant_key(attn):
    """A key whose score exceeds every other by >= 1000 takes all the weight."""
    gen = torch.Generator().manual_seed(17)
    q = torch.ones((1, 1, 2, 4), dtype=F64)
    k = torch.randn((1, 1, 6, 4), generator=gen, dtype=F64)
    k[0, 0, 4] = 600.0
    v = torch.randn((1, 1, 6, 3), generator=gen, dtype=F64)
    o, lse = attn(q, k, v, SCALE)
    _close(o, v[:, :, 4:5].expand(1, 1, 2, 3), 1e-14, "dominant_key O")
    _close(lse, torch.full((1, 1, 2), SCALE * 2400.0, dtype=F64), 1e-9, "dominant_key lse")


def pin_brute_force(attn):
    """Scalar loops with math.exp on a 3-query, 5-key case (D=4, Dv=2)."""
    gen = torch.Generator().manual_seed(18)
    q = torch.randn((1, 1, 3, 4), generator=gen, dtype=F64) * 2
    k = torch.randn((1, 1, 5, 4), generator=gen, dtype=F64) * 2
    v = torch.randn((1, 1, 5, 2), generator=gen, dtype=F64)
    o, lse = attn(q, k, v, SCALE)
    Q, K, V = q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist()
    for i in range(3):
        w = [math.exp(SCALE * sum(Q[i][d] * K[j][d] for d in range(4))) for j in range(5)]
        z = sum(w)
        for e in range(2):
            want = sum(w[j] * V[j][e] for j in range(5)) / z
            _close(o[0, 0, i, e], want, 1e-13, f"brute_force O[{i},{e}]")
        _close(lse[0, 0, i], math.log(z), 1e-13, f"brute_force lse[{i}]")


def pin_sdpa(attn):
    """torch's scaled_dot_product_attention and logsumexp, float64 on the CPU."""
    gen = torch.Generator().manual_seed(19)
    q = torch.randn((2, 3, 33, 16), generator=gen, dtype=F64)
    k = torch.randn((2, 3, 47, 16), generator=gen, dtype=F64) * 3
    v = torch.randn((2, 3, 47, 8), generator=gen, dtype=F64)
    o, lse = attn(q, k, v, SCALE)
    want = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=SCALE)
    _close(o, want, 1e-12, "sdpa O")
    want_lse = torch.logsumexp(torch.matmul(q, k.transpose(-1, -2).contiguous()) * SCALE, dim=-1)
    _close(lse, want_lse, 1e-12, "sdpa lse")


def _f32(x: float) -> float:
    """x rounded to the nearest float32 (the scale the kernel receives)."""
    return struct.unpack("f", struct.pack("f", x))[0]


def pin_inexact_scale(attn):
    """Scale 0.1 is not a float32 value; the contract is that the scores use
    its float32 rounding sigma = 0.100000001490116... Two keys 0 and a with
    q = 1 (D = 1): the weight of key 1 is sigmoid(sigma a) and lse =
    softplus(sigma a). At a = 10 the unrounded scale moves O by ~5e-9, at
    a = 1e6 it moves lse by ~1.5e-3; both far above the tolerances."""
    scale = 0.1
    sigma = _f32(scale)
    assert sigma != scale
    v0, v1 = 0.25, -1.5
    for a, o_tol, lse_tol in ((10.0, 1e-13, 1e-13), (1e6, 1e-13, 1e-9)):
        q = _t([[[[1.0]]]])
        k = _t([[[[0.0], [a]]]])
        v = _t([[[[v0], [v1]]]])
        o, lse = attn(q, k, v, scale)
        x = sigma * a
        w1 = 1.0 / (1.0 + math.exp(-x))
        _close(o, _t([[[[v0 + (v1 - v0) * w1]]]]), o_tol, f"inexact_scale O a={a}")
        _close(lse, _t([[[x + math.log1p(math.exp(-x))]]]), lse_tol, f"inexact_scale lse a={a}")


ALL_PINS = [pin_two_keys, pin_orthogonal_keys, pin_q_zero, pin_identical_keys, pin_key_shift,
            pin_permutation, pin_affine_v, pin_single_key, pin_dominant_key, pin_brute_force,
            pin_sdpa, pin_inexact_scale]


# ---- pins of the probability matrix: probs(q, k, scale) -> P [B, H, S_q, S_k] ----

def pin_probs_two_keys(probs):
    """q = 1 (D = 1), keys 0 and a: P = (1 - w, w) with w = sigmoid(sigma a),
    for an exact scale (0.5) and an inexact one (0.1, sigma its float32
    rounding), including sigma a = 1000 where exp without the max overflows."""
    for scale in (0.5, 0.1):
        sigma = _f32(scale)
        for a in (0.0, 1.0, -3.0, 10.0, 2000.0 if scale == 0.5 else 10000.0):
            p = probs(_t([[[[1.0]]]]), _t([[[[0.0], [a]]]]), scale)
            x = sigma * a
            w1 = 1.0 / (1.0 + math.exp(-x)) if x >= 0 else math.exp(x) / (1.0 + math.exp(x))
            _close(p, _t([[[[1.0 - w1, w1]]]]), 1e-15, f"probs two_keys scale={scale} a={a}")


def pin_probs_orthogonal_keys(probs):
    """K = c I (4 keys, D = 4), query i = unit vector pi(i): row i has
    e^(sigma c) / (e^(sigma c) + 3) at column pi(i) and 1 / (e^(sigma c) + 3)
    elsewhere. A transposed P (softmax over queries) differs, since pi is a
    cycle and the rows are not symmetric."""
    c = 3.0
    pi = [1, 2, 3, 0]
    q = torch.zeros((1, 1, 4, 4), dtype=F64)
    for i, j in enumerate(pi):
        q[0, 0, i, j] = 1.0
    k = (c * torch.eye(4, dtype=F64)).reshape(1, 1, 4, 4)
    # a fifth key that no query sees (zero score) makes P non-square
    k = torch.cat([k, torch.zeros((1, 1, 1, 4), dtype=F64)], dim=2)
    p = probs(q, k, SCALE)
    big = math.exp(SCALE * c)
    want = torch.full((4, 5), 1.0 / (big + 4.0), dtype=F64)
    for i in range(4):
        want[i, pi[i]] = big / (big + 4.0)
    _close(p[0, 0], want, 1e-15, "probs orthogonal_keys")


def pin_probs_weighted_mean(probs):
    """P.V equals the brute-force softmax-weighted mean (scalar math.exp loops)."""
    gen = torch.Generator().manual_seed(20)
    q = torch.randn((1, 1, 3, 4), generator=gen, dtype=F64) * 2
    k = torch.randn((1, 1, 6, 4), generator=gen, dtype=F64) * 2
    v = torch.randn((1, 1, 6, 2), generator=gen, dtype=F64)
    p = probs(q, k, 0.3)
    sigma = _f32(0.3)
    Q, K, V = q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist()
    pv = p[0, 0] @ v[0, 0]
    for i in range(3):
        w = [math.exp(sigma * sum(Q[i][d] * K[j][d] for d in range(4))) for j in range(6)]
        z = sum(w)
        for e in range(2):
            _close(pv[i, e], sum(w[j] * V[j][e] for j in range(6)) / z, 1e-13, f"probs weighted_mean [{i},{e}]")


PROB_PINS = [pin_probs_two_keys, pin_probs_orthogonal_keys, pin_probs_weighted_mean]
