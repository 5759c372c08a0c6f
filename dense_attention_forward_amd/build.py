"""Compile the gfx950 attention library in-tree with hipcc.

Produces ``dense_attention_forward_amd/libattn_fwd.so`` from the HIP kernel
and the C-ABI host code. Run ``python -m dense_attention_forward_amd.build``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libattn_fwd.so"

SOURCES = [CSRC / "attn_fwd_kernel.hip", CSRC / "attn_fwd_abi.cpp", CSRC / "attn_mfma_rate.hip"]
HEADERS = [ROOT / "include" / "attn_fwd.h", ROOT / "include" / "attn_mfma_rate.h", CSRC / "attn_fwd_launch.h"]

ARCH = "gfx950"
# Packed-FP32 VALU forms are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def command(out: Path = LIB, extra: list[str] | None = None) -> list[str]:
    return ([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-fvisibility=hidden", "-Wall", "-I", str(ROOT / "include"), "-I", str(CSRC)] + DEVICE_FLAGS
            + (extra or []) + [str(s) for s in SOURCES] + ["-o", str(out)])


def build(verbose: bool = False) -> Path:
    """Always recompiles; writes to a temp file and renames so a failed build
    never leaves a half-written library behind."""
    tmp = LIB.with_suffix(".so.tmp")
    cmd = command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n")
        noise = ("packed-fp32-ops", "not a recognized feature")
        sys.stderr.write("".join(l + "\n" for l in res.stderr.splitlines()
                                 if not any(s in l for s in noise)))
    if res.returncode != 0:
        tmp.unlink(missing_ok=True)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
