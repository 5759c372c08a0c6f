"""The software exp2 of the PAIR256_EXP2EMU kernel variant: its float32
polynomial coefficients (read from the kernel source) approximate 2**f on
[0, 1] to the stated relative error, checked against numpy's exp2 in
float64 on a dense grid, and the kernel's reconstruction (clamp at -127,
split into floor and fraction, Horner cubic by fused multiply-add, scale by
2**n), emulated step by step in float32, keeps that bound over the whole
range of arguments the kernel can see: any finite value up to the rebase
threshold of 16. No GPU needed."""
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


def _threshold():
    m = re.search(r"constexpr float kRebaseLog2 = ([0-9.]+)f;", SRC.read_text())
    return float(m.group(1))


def _fma32(a, b, c):
    """float32 fused multiply-add: the float32 product is exact in float64."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(F32)


def _kernel_exp2(c, x):
    """The kernel's exp2_poly, step by step in float32."""
    xc = np.maximum(x.astype(F32), F32(-127.0))
    n = np.floor(xc)
    f = (xc - n).astype(F32)
    p = _fma32(np.full_like(f, c[3]), f, np.full_like(f, c[2]))
    p = _fma32(p, f, np.full_like(f, c[1]))
    p = _fma32(p, f, np.full_like(f, c[0]))
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
    """x = s*c - kept lies below the rebase threshold (16); in [-126, 16]
    the float32 emulation of the kernel's steps stays within the bound."""
    c = _coeffs()
    top = _threshold()
    assert top == 16.0
    x = np.linspace(-126.0, top, 1_000_001).astype(F32)
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
