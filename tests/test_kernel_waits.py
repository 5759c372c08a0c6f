"""Static check of the eight-wave kernels' explicit LDS waits (no GPU).

The MFMA phase issues its LDS operand reads as inline assembly and waits for
them with hand-computed `s_waitcnt lgkmcnt(N)` (one wait per group of
fragments). A wrong N would let an MFMA read an operand register before its
LDS read has returned, which no test of the results is sure to catch (the
data often lands in time anyway). This test compiles the kernels to
assembly and replays each kernel's instruction stream in program order:
LDS reads of one wave complete in issue order, so after `lgkmcnt(N)` all
but the last N outstanding reads have landed. It fails if any instruction
reads or writes a register that an outstanding LDS read will still write."""
import re

import pytest

from tests.test_kernel_asm import _asm, _regs


def _operand_regs(ins: str) -> set:
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return set()
    out = set()
    for tok in re.split(r"[,\s]+", parts[1]):
        out |= _regs(tok)
    return out


def _lgkm_limit(ins: str):
    m = re.search(r"lgkmcnt\((\d+)\)", ins)
    return int(m.group(1)) if m else None


def check_waits(lines):
    """Replay instructions; return a list of violations (instruction, pending registers)."""
    pending = []  # outstanding LDS reads in issue order: sets of destination registers
    bad = []
    for ins in lines:
        op = ins.split()[0]
        if op == "s_waitcnt":
            n = _lgkm_limit(ins)
            if n is not None:
                while len(pending) > n:
                    pending.pop(0)
            continue
        regs = _operand_regs(ins)
        busy = set().union(*pending) if pending else set()
        if op.startswith("ds_read") or op.startswith("ds_load"):
            dst = _regs(ins.split(None, 1)[1].split(",")[0].strip())
            if (regs - dst) & busy or dst & busy:
                bad.append((ins, sorted(busy & regs)))
            pending.append(dst)
            continue
        if op.startswith("s_memtime") or op.startswith("s_load") or op.startswith("s_buffer_load"):
            pending.append(set())  # scalar memory also counts in lgkmcnt
            continue
        if regs & busy:
            bad.append((ins, sorted(regs & busy)))
    return bad


def _kernel_lines(text: str, name_part: str):
    start = text.index(name_part)
    body = text[start:text.index(".Lfunc_end", start)]
    out = []
    for line in body.splitlines():
        s = line.strip()
        if s and not s.startswith((";", ".")) and not s.endswith(":"):
            out.append(s)
    return out


def test_checker_flags_an_early_read():
    lines = ["ds_read_b128 v[10:13], v1", "ds_read_b128 v[14:17], v1 offset:64",
             "s_waitcnt lgkmcnt(1)",
             "v_mfma_f32_16x16x32_bf16 v[0:3], v[10:13], v[20:23], v[0:3]",
             "v_mfma_f32_16x16x32_bf16 v[4:7], v[14:17], v[20:23], v[4:7]"]
    bad = check_waits(lines)
    assert len(bad) == 1 and "v[14:17]" in bad[0][0]
    ok = lines[:3] + [lines[3], "s_waitcnt lgkmcnt(0)", lines[4]]
    assert check_waits(ok) == []
    # a read into a register that an earlier read still owns is flagged too
    assert len(check_waits(["ds_read_b128 v[10:13], v1", "ds_read_b128 v[12:15], v1"])) == 1


@pytest.mark.parametrize("kernel", ["pingpong_kernelILi128ELi2ELi0E", "pingpong_kernelILi128ELi2ELi4E",
                                    "pingpong_kernelILi128ELi1ELi0E"])
def test_mfma_phase_waits_cover_every_operand(tmp_path, kernel):
    text = _asm(tmp_path)
    lines = _kernel_lines(text, kernel)
    assert sum(l.startswith("ds_read_b64_tr_b16") for l in lines) >= 64
    bad = check_waits(lines)
    assert bad == [], bad[:5]
