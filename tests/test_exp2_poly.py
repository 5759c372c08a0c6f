"""The software exp2 of the PAIR256_EXP2EMU kernel variant: its float32
polynomial coefficients (read from the kernel source) approximate 2**f on
[0, 1] to the stated relative error, checked against numpy's exp2 in
float64 on a dense grid, and the kernel's reconstruction (clamp to
[-127, 128], split into floor and fraction, Horner cubic by fused
multiply-add, scale by 2**n), emulated step by step in float32, keeps that
bound wherever the kernel keeps the result (arguments below 1, against its
raised base), gives at most 2^-126 below -126, and gives at least 2 (the
exponent bit of the kernel's rebase test) for every argument from 1 up,
Inf included. No GPU needed."""
import re
from pathlib import Path

import numpy as np

SRC = Path(__file__).resolve().parent.parent / "dense_attention_forward_amd" / "csrc" / "attn_fwd_kernel.hip"
F32 = np.float32


def _coeffs():
    text = SRC.read_text()
    c = {int(k): float(v) for k, v in re.findall(r"constexpr float kExp2C(\d) = ([0-9.eE+-]+)f;", text)}
    assert sorted(c) == [0, 1, 2, 3]
    return np.array([c[k] for k in range(4)], dtype=F32)


def _bit_threshold():
    m = re.search(r"constexpr float kBitRebaseLog2 = ([0-9.]+)f;", SRC.read_text())
    return float(m.group(1))


def _fma32(a, b, c):
    """float32 fused multiply-add: the float32 product is exact in float64."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(F32)


def _kernel_exp2(c, x):
    """The kernel's exp2_poly, step by step in float32."""
    xc = np.clip(x.astype(F32), F32(-127.0), F32(128.0))
    n = np.floor(xc)
    f = (xc - n).astype(F32)
    p = _fma32(np.full_like(f, c[3]), f, np.full_like(f, c[2]))
    p = _fma32(p, f, np.full_like(f, c[1]))
    p = _fma32(p, f, np.full_like(f, c[0]))
    with np.errstate(over="ignore"):
        return np.ldexp(p, n.astype(np.int32)).astype(F32)


def _poly(c, f):
    c = c.astype(np.float64)
    return ((c[3] * f + c[2]) * f + c[1]) * f + c[0]


def test_relative_error_on_unit_interval():
    c = _coeffs()
    assert c[0] == 1.0  # integer arguments are exact
    f = np.linspace(0.0, 1.0, 2_000_001)
    rel = np.abs(_poly(c, f) - np.exp2(f)) / np.exp2(f)
    assert rel.max() <= 1.0e-4


def test_reconstruction_over_the_range_used():
    """The P the kernel keeps has x = s*c - kept below 1 (its base is raised
    by the threshold less one); in [-126, 1] the float32 emulation of the
    kernel's steps stays within the bound. [1, 16] is checked as well."""
    c = _coeffs()
    assert _bit_threshold() >= 1.0
    x = np.linspace(-126.0, 16.0, 1_000_001).astype(F32)
    approx = _kernel_exp2(c, x).astype(np.float64)
    exact = np.exp2(x.astype(np.float64))
    rel = np.abs(approx - exact) / exact
    assert rel.max() <= 1.0e-4


def test_far_negative_arguments_give_tiny_values():
    """Any finite argument below -126, down to -2^127, gives a finite,
    non-negative value of at most 2^-126 (the exponent unit returns 0 there)."""
    c = _coeffs()
    x = -np.exp2(np.linspace(np.log2(126.0), 127.0, 100_001)).astype(F32)
    x = np.concatenate([x, np.array([-126.5, -127.0, -1e30, -3.4e38], dtype=F32)])
    y = _kernel_exp2(c, x)
    assert np.isfinite(y).all()
    assert (y >= 0).all() and (y <= 2.0 ** -126).all()


def _bf16_bits(y):
    """Round-to-nearest-even float32 -> bf16 bit patterns (as the kernel's
    v_cvt_pk_bf16_f32), NaN aside."""
    b = y.astype(F32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint32)


def test_arguments_from_one_up_set_the_rebase_bit():
    """The eight-wave kernel computes P against its kept base first and
    rebases a row when the top exponent bit of some bf16 P is set (P >= 2).
    Every argument from 1 up to the largest float, and +Inf, must set it in
    the software exp2 too; arguments just below 1 may round up to 2, which
    only costs a redundant rebase test."""
    c = _coeffs()
    x = np.concatenate([np.linspace(1.0, 130.0, 200_001), np.exp2(np.linspace(7.0, 127.9, 10_001)),
                        np.array([np.finfo(np.float32).max, np.inf])]).astype(F32)
    y = _kernel_exp2(c, x)
    assert not np.isnan(y).any()
    assert (y >= 2.0).all()
    assert (y[x >= 128.0] == np.inf).all()
    assert ((_bf16_bits(y) & 0x4000) != 0).all()
    below = np.linspace(-126.0, 0.99, 100_001).astype(F32)
    assert ((_bf16_bits(_kernel_exp2(c, below)) & 0x4000) == 0).all()
