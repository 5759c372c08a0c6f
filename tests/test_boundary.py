"""The C-ABI library: it loads, exports every declared symbol, and its
host-side validation returns the documented codes (no GPU needed: nothing
here launches a kernel or touches device memory)."""
import math
import re
import subprocess
from pathlib import Path

import pytest
import torch

ROOT = Path(__file__).resolve().parent.parent
HEADERS = sorted((ROOT / "include").glob("*.h"))


def _ensure_built():
    from dense_attention_forward_amd import build as b
    if not b.LIB.exists():
        b.build()
    return b.LIB


@pytest.fixture(scope="module")
def lib():
    _ensure_built()
    import dense_attention_forward_amd as daf
    return daf


def _declared_functions():
    names = []
    for h in HEADERS:
        text = h.read_text()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M):
            if m.group(1) not in ("if", "defined"):
                names.append(m.group(1))
    return names


def test_header_declares_the_boundary():
    assert set(_declared_functions()) >= {"attn_fwd", "attn_fwd_check", "attn_status_str",
                                          "attn_fwd_variant", "attn_fwd_pick"}


def _exported_functions(path):
    """Names of the functions the shared library exports (defined, dynamic, text)."""
    out = subprocess.run(["nm", "-D", "--defined-only", str(path)], capture_output=True,
                         text=True, check=True).stdout
    return {line.split()[-1] for line in out.splitlines()
            if line.strip() and line.split()[-2] in ("T", "W")}


def test_every_declared_symbol_is_exported(lib):
    exported = _exported_functions(lib.LIB_PATH)
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib.lib(), name) is not None


def test_only_declared_symbols_are_exported(lib):
    """The library is built with hidden visibility: nothing but the C ABI of
    the headers (no C++ internals) is visible to a client."""
    assert _exported_functions(lib.LIB_PATH) == set(_declared_functions())


# Fake, aligned, non-overlapping "device" addresses: only compared, never dereferenced.
B, H, S, D = 2, 3, 256, 128
NB = B * H * S * D * 2
Q, K, V, O, L = (0x10000000 + i * 0x1000000 for i in range(5))
SC = 1.0 / math.sqrt(128)


def _check(lib, q=Q, k=K, v=V, o=O, l=L, b=B, h=H, s=S, d=D, scale=SC):
    return lib.check(q, k, v, o, l, b, h, s, d, scale)


def test_check_ok(lib):
    assert _check(lib) == 0


# Far-apart fake addresses for huge shapes (2^30 rows of 256 bytes each = 256 GiB per tensor).
FAR = [(i + 1) << 40 for i in range(5)]


def test_grid_limit_per_variant(lib):
    """B*H*S = 2^30 rows: one 128-row tile per 4-wave workgroup needs 2^31
    threads, while the pairs of 64-row tiles of PAIR128 (8 waves per 128
    rows) would need 2^32, beyond the launch limit: a forced PAIR128 call
    is refused as a shape error before any launch, and the library's own
    pick (which falls back from PAIR256, also 2^32 threads at S = 128)
    accepts the shape."""
    q, k, v, o, l = FAR
    b, h, s = 1, 1 << 23, 128
    assert lib.check(q, k, v, o, l, b, h, s, D, SC) == 0
    assert lib.pick(b, h, s) == lib.VARIANT_TILE128
    for variant in (lib.VARIANT_PAIR128, lib.VARIANT_PAIR256, lib.VARIANT_PAIR256_EXP2EMU):
        assert lib.attn_fwd_raw(q, k, v, o, l, b, h, s, D, SC, 0, variant=variant) == 2
    # twice the rows: every variant would need 2^32 threads or more
    assert lib.check(q, k, v, o, l, 2, h, s, D, SC) == 2
    # at S = 256 PAIR256 needs no more threads than TILE128 and is kept
    assert lib.pick(1, 1 << 22, 256) == lib.VARIANT_PAIR256
    assert lib.check(q, k, v, o, l, 1, 1 << 22, 256, D, SC) == 0


@pytest.mark.parametrize("arg", ["q", "k", "v", "o", "l"])
def test_check_null(lib, arg):
    assert _check(lib, **{arg: 0}) == 1


@pytest.mark.parametrize("kw", [dict(d=64), dict(d=256), dict(s=100), dict(s=0), dict(s=-128), dict(s=64),
                                dict(b=0), dict(h=0), dict(b=-1), dict(b=65536, h=65536, s=128)])
def test_check_shape(lib, kw):
    assert _check(lib, **kw) == 2


@pytest.mark.parametrize("arg", ["q", "k", "v", "o", "l"])
def test_check_align(lib, arg):
    base = {"q": Q, "k": K, "v": V, "o": O, "l": L}[arg]
    assert _check(lib, **{arg: base + 4}) == 3


@pytest.mark.parametrize("scale", [0.0, -0.1, float("nan"), float("inf"), -float("inf")])
def test_check_scale(lib, scale):
    assert _check(lib, scale=scale) == 4


@pytest.mark.parametrize("kw", [dict(o=Q), dict(o=K + 4096), dict(l=V + NB - 16), dict(l=O + 16),
                                dict(o=L - NB + 16)])
def test_check_overlap(lib, kw):
    assert _check(lib, **kw) == 5


def test_adjacent_buffers_do_not_overlap(lib):
    assert _check(lib, o=Q + NB) == 0
    assert _check(lib, l=O + NB) == 0


def test_status_strings(lib):
    for code in range(8):
        s = lib.status_str(code)
        assert isinstance(s, str) and s
    assert lib.status_str(0) == "ok"
    assert lib.status_str(99) == "unknown status"


def test_attn_fwd_rejects_before_launch(lib):
    """The launching entry point validates first; a bad call returns the code
    without any HIP call, so this runs without a GPU."""
    assert lib.attn_fwd_raw(Q, K, V, O, L, B, H, S, 64, SC, 0) == 2
    assert lib.attn_fwd_raw(0, K, V, O, L, B, H, S, D, SC, 0) == 1
    assert lib.attn_fwd_raw(Q, K, V, O, L, B, H, S, D, -1.0, 0) == 4


def test_python_wrapper_rejects_bad_tensors(lib):
    q = torch.zeros((1, 1, 128, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        lib.forward(q, q, q)  # CPU tensors are rejected before any call
    with pytest.raises(ValueError):
        lib.forward(q.float(), q, q)


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    from dense_attention_forward_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", tmp_path / "absent.so")
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def test_variant_rejected_before_launch(lib):
    for bad in (-1, 5, 99):
        assert lib.attn_fwd_raw(Q, K, V, O, L, B, H, S, D, SC, 0, variant=bad) == 7
    # a valid variant with bad arguments still reports the argument error
    assert lib.attn_fwd_raw(Q, K, V, O, L, B, H, S, 64, SC, 0, variant=2) == 2


def test_pick(lib):
    # launches of a few workgroups keep one 128-row tile per workgroup
    assert lib.pick(1, 1, 256) == lib.VARIANT_TILE128
    assert lib.pick(1, 1, 1024) == lib.VARIANT_TILE128
    # below a full round of 256-row workgroups: pairs of 64-row tiles
    assert lib.pick(1, 4, 1024) == lib.VARIANT_PAIR128
    assert lib.pick(1, 1, 8192) == lib.VARIANT_PAIR128
    assert lib.pick(2, 16, 1024) == lib.VARIANT_PAIR128
    assert lib.pick(1, 16, 2048) == lib.VARIANT_PAIR128
    assert lib.pick(2, 8, 1024) == lib.VARIANT_PAIR128
    # one full round of 256-row workgroups and more
    assert lib.pick(2, 16, 2048) == lib.VARIANT_PAIR256
    assert lib.pick(4, 16, 1024) == lib.VARIANT_PAIR256
    # the 4K/8K/16K workloads fill the GPU with tile pairs
    assert lib.pick(4, 16, 4096) == lib.VARIANT_PAIR256
    assert lib.pick(2, 16, 8192) == lib.VARIANT_PAIR256
    assert lib.pick(1, 16, 16384) == lib.VARIANT_PAIR256


def test_mfma_rate_rejects_before_launch(lib):
    """The MFMA-rate probe validates its arguments before any HIP call."""
    r = lib.lib().attn_mfma_rate
    assert r(0, L, 8, 10, 0) == 1
    assert r(Q, 0, 8, 10, 0) == 1
    assert r(Q + 8, L, 8, 10, 0) == 3
    assert r(Q, L + 2, 8, 10, 0) == 3
    assert r(Q, L, 0, 10, 0) == 2
    assert r(Q, L, 8, 0, 0) == 2
    assert r(Q, L, 2 ** 30, 10, 0) == 2
