"""Static checks of the generated gfx950 assembly (no GPU).

The compiler's hazard checks do not see an MFMA written as inline assembly.
A VALU write to a register that such an MFMA reads a few instructions later
then goes without the wait states the hardware needs, and the MFMA may read
a stale value (this happened once with a constant operand the compiler
rebuilt with v_mov right before each use). This test compiles the kernels to
assembly and checks that no VALU instruction writes a register read by an
inline-assembly MFMA within the next few instructions, that no other
instruction reads or writes an inline-assembly MFMA's result within the
wait states its latency needs, and that the eight-wave kernels neither spill
nor use scratch."""
import re
import subprocess
from pathlib import Path

import pytest

from dense_attention_forward_amd import build

WINDOW = 6  # instructions before each inline-assembly MFMA that are checked


def _asm(tmp_path: Path) -> str:
    out = tmp_path / "kernel.s"
    cmd = [build.hipcc(), f"--offload-arch={build.ARCH}", "-O3", "-std=c++17", "-I",
           str(build.ROOT / "include"), "-I", str(build.CSRC)] + build.DEVICE_FLAGS + [
        "--cuda-device-only", "-S", "-o", str(out), str(build.CSRC / "attn_fwd_kernel.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.fail(res.stderr[-2000:])
    return out.read_text()


def _regs(tok: str) -> set:
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


def _instructions(text: str):
    """(from_inline_asm, instruction) in program order."""
    in_asm = False
    for line in text.splitlines():
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
        elif s.startswith(";;#ASMEND"):
            in_asm = False
        elif s and not s.startswith((";", ".")) and not s.endswith(":"):
            yield in_asm, s


def _hazards(text: str):
    insts = list(_instructions(text))
    found = []
    for i, (in_asm, s) in enumerate(insts):
        if not (in_asm and s.startswith("v_mfma")):
            continue
        ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
        srcs = set().union(*(_regs(o) for o in ops[1:]))
        for _, p in insts[max(0, i - WINDOW):i]:
            if p.startswith("v_") and not p.startswith("v_mfma"):
                dst = _regs(p.split(None, 1)[1].split(",")[0].strip())
                if dst & srcs:
                    found.append(f"{p}  ->  {s}")
    return found


# Wait states between an 8-pass MFMA (v_mfma_f32_16x16x32_bf16) writing a
# register and any other instruction reading or writing it.
MFMA_RESULT_WAIT = 11


def _wait_states(s: str) -> int:
    m = re.fullmatch(r"s_nop\s+(\d+)", s)
    return int(m.group(1)) + 1 if m else 1


def _result_hazards(text: str):
    """Inline-assembly MFMA results used by a non-MFMA instruction before
    MFMA_RESULT_WAIT wait states have passed (in program order)."""
    insts = list(_instructions(text))
    found = []
    for i, (in_asm, s) in enumerate(insts):
        if not (in_asm and s.startswith("v_mfma")):
            continue
        dst = _regs(s.split(None, 1)[1].split(",")[0].strip())
        waited = 0
        for _, p in insts[i + 1:]:
            if waited >= MFMA_RESULT_WAIT:
                break
            if not p.startswith("v_mfma") and not p.startswith("s_"):
                parts = p.split(None, 1)
                ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
                used = set().union(set(), *(_regs(o) for o in ops))
                if used & dst:
                    found.append(f"{s}  ->  {p} after {waited} wait states")
                    break
            waited += _wait_states(p)
    return found


def test_checker_flags_a_planted_hazard():
    text = "\n".join(["\tv_mov_b32_e32 v10, s4", ";;#ASMSTART",
                      "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[8:11], v[12:15], v[0:3]", ";;#ASMEND"])
    assert len(_hazards(text)) == 1
    text = "\n".join(["\tv_mov_b32_e32 v20, s4", ";;#ASMSTART",
                      "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[8:11], v[12:15], v[0:3]", ";;#ASMEND"])
    assert _hazards(text) == []


def test_result_checker_flags_an_early_read():
    mfma = ["\t;;#ASMSTART", "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[8:11], v[12:15], v[0:3]", "\t;;#ASMEND"]
    early = mfma + ["\ts_nop 7", "\tv_mul_f32_e32 v20, v5, v2"]
    assert len(_result_hazards("\n".join(early))) == 1
    waited = mfma + ["\ts_nop 7", "\ts_nop 2", "\tv_mul_f32_e32 v20, v5, v2"]
    assert _result_hazards("\n".join(waited)) == []
    other = mfma + ["\tv_mul_f32_e32 v20, v5, v6"]
    assert _result_hazards("\n".join(other)) == []


def test_no_early_use_of_an_asm_mfma_result(tmp_path):
    text = _asm(tmp_path)
    assert _result_hazards(text) == []


def test_no_valu_write_feeds_an_asm_mfma(tmp_path):
    text = _asm(tmp_path)
    assert text.count("v_mfma_f32_16x16x32_bf16") > 100
    assert _hazards(text) == []


def test_eight_wave_kernels_do_not_spill(tmp_path):
    text = _asm(tmp_path)
    checked = 0
    for name, body in re.findall(r"\.name:\s+(\S+)(.*?)(?=\.name:|\Z)", text, re.S):
        if "pingpong" not in name:
            continue
        assert re.search(r"\.vgpr_spill_count:\s+0\b", body), name
        assert re.search(r"\.private_segment_fixed_size:\s+0\b", body), name
        checked += 1
    assert checked == 3
