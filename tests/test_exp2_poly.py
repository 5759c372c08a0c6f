"""The software exp2 of the PAIR256_EXP2EMU kernel variant: its float32
polynomial coefficients (read from the kernel source) approximate 2**f on
[0, 1] to the stated relative error, checked against numpy's exp2 in
float64 on a dense grid, and the reconstruction 2**n * p(f) keeps that
bound across exponents. No GPU needed."""
import re
from pathlib import Path

import numpy as np

SRC = Path(__file__).resolve().parent.parent / "dense_attention_forward_amd" / "csrc" / "attn_fwd_kernel.hip"


def _coeffs():
    text = SRC.read_text()
    c = {int(k): float(v) for k, v in re.findall(r"constexpr float kExp2C(\d) = ([0-9.eE+-]+)f;", text)}
    assert sorted(c) == [0, 1, 2, 3]
    return np.array([c[k] for k in range(4)], dtype=np.float32).astype(np.float64)


def _poly(c, f):
    return ((c[3] * f + c[2]) * f + c[1]) * f + c[0]


def test_relative_error_on_unit_interval():
    c = _coeffs()
    assert c[0] == 1.0  # integer arguments are exact
    f = np.linspace(0.0, 1.0, 2_000_001)
    rel = np.abs(_poly(c, f) - np.exp2(f)) / np.exp2(f)
    assert rel.max() <= 1.0e-4


def test_reconstruction_over_the_range_used():
    """x = s*c - kept lies in [-inf, 8] (lazy rescale bound); 2**floor(x) *
    p(x - floor(x)) must stay within the bound everywhere in [-126, 8]."""
    c = _coeffs()
    x = np.linspace(-126.0, 8.0, 1_000_001)
    n = np.floor(x)
    approx = np.ldexp(_poly(c, x - n), n.astype(np.int64))
    rel = np.abs(approx - np.exp2(x)) / np.exp2(x)
    assert rel.max() <= 1.0e-4
