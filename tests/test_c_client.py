"""The library from plain C: tests/c_abi/attn_c_client.c is compiled with
gcc as C99 against include/attn_fwd.h and the HIP runtime's C API, and run.
The host checks need no GPU; the GPU case writes seeded inputs, lets the C
client run attn_fwd, and compares its O and LSE with the oracle."""
import shutil
import struct
import subprocess
from pathlib import Path

import numpy as np
import pytest
import torch

import oracle
from workloads import DEFAULT_SCALE, make_random

ROOT = Path(__file__).resolve().parent.parent
PKG = ROOT / "dense_attention_forward_amd"
SRC = Path(__file__).resolve().parent / "c_abi" / "attn_c_client.c"
ROCM = Path("/opt/rocm")


def _compile(tmp_path: Path) -> Path:
    from dense_attention_forward_amd import build as b
    if not b.LIB.exists():
        b.build()
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.fail("gcc is required to build the C client")
    exe = tmp_path / "attn_c_client"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", str(ROCM / "include"), "-I", str(ROOT / "include"), str(SRC),
           "-L", str(PKG), "-lattn_fwd", "-L", str(ROCM / "lib"), "-lamdhip64",
           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{ROCM / 'lib'}", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def test_c_client_host_checks(tmp_path):
    exe = _compile(tmp_path)
    res = subprocess.run([str(exe), "host"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failure(s)" in res.stdout


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,S", [(1, 2, 384), (1, 32, 4096)])
def test_c_client_runs_attention(tmp_path, B, H, S):
    """S = 384 at H = 2 takes the four-wave kernel, S = 4096 at H = 32 the eight-wave PAIR256."""
    print(f"case C client B={B} H={H} S={S}", flush=True)
    exe = _compile(tmp_path)
    q, k, v = make_random(B, H, S, 128, seed=31)
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(struct.pack("<4if", B, H, S, 128, DEFAULT_SCALE))
        for t in (q, k, v):
            f.write(t.view(torch.int16).numpy().tobytes())
    res = subprocess.run([str(exe), "run", str(inp), str(out)], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    n, rows = B * H * S * 128, B * H * S
    raw = out.read_bytes()
    assert len(raw) == 2 * n + 4 * rows
    o = torch.from_numpy(np.frombuffer(raw[:2 * n], dtype=np.int16).copy()).view(torch.bfloat16)
    lse = torch.from_numpy(np.frombuffer(raw[2 * n:], dtype=np.float32).copy())
    o = o.reshape(B, H, S, 128).double()
    lse = lse.reshape(B, H, S).double()
    if S <= 512:
        o_ref, lse_ref = oracle.attention(q, k, v, DEFAULT_SCALE)
        err = (o - o_ref).abs()
        rel = ((lse - lse_ref).abs() / lse_ref.abs().clamp_min(1.0)).max().item()
    else:
        picks = [(0, h, r) for h in range(H) for r in (0, 1, 127, 128, S // 2, S - 1)]
        o_ref, lse_ref = oracle.attention_rows(q, k, v, DEFAULT_SCALE, picks)
        idx = tuple(torch.tensor(x) for x in zip(*picks))
        err = (o[idx] - o_ref).abs()
        rel = ((lse[idx] - lse_ref).abs() / lse_ref.abs().clamp_min(1.0)).max().item()
    print(f"  O max-abs {err.max().item():.3e} mean-abs {err.mean().item():.3e} LSE max-rel {rel:.3e}",
          flush=True)
    assert err.max().item() <= 2e-2 and err.mean().item() <= 2e-3 and rel <= 1e-3
