"""Static check of the eight-wave kernels' explicit LDS waits (no GPU).

The MFMA phase issues its LDS operand reads as inline assembly and waits for
them with hand-computed `s_waitcnt lgkmcnt(N)` (one wait per group of
fragments). A wrong N would let an MFMA read an operand register before its
LDS read has returned, which no test of the results is sure to catch (the
data often lands in time anyway). This test compiles the kernels to
assembly and replays each kernel's instructions along every path of its
control-flow graph (the reads of one loop iteration may still be in flight
when the next begins): LDS reads of one wave complete in issue order, so
after `lgkmcnt(N)` all but the last N outstanding reads have landed. It
fails if any instruction reads or writes a register that an outstanding LDS
read will still write, which also catches a read whose address register an
earlier read of the same wave is about to overwrite."""
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


_LGKM_MAX = 15
_BRANCH = re.compile(r"^s_(c?branch\w*)\s+(\S+)")


def _blocks(text: str, name_part: str):
    """Basic blocks of one kernel: (label, [instructions], [successor labels])."""
    start = text.index(name_part)
    body = text[start:text.index(".Lfunc_end", start)]
    blocks, cur = [], None
    n = 0

    def new_block(label):
        nonlocal cur
        cur = [label, [], []]
        blocks.append(cur)

    new_block("<entry>")
    for line in body.splitlines()[1:]:
        s = line.strip()
        if not s or s.startswith(";"):
            continue
        m = re.match(r"^([.\w$]+):", s)
        if m and not s.startswith(".Lfunc"):
            new_block(m.group(1))
            continue
        if s.startswith("."):
            continue
        cur[1].append(s)
        op = s.split()[0]
        m = _BRANCH.match(s)
        if m or op in ("s_endpgm", "s_setpc_b64"):
            if m:
                cur[2].append(m.group(2))
            cur.append(op)  # terminator
            n += 1
            new_block(f"<after {n}>")
    # fallthrough edges
    for i, b in enumerate(blocks):
        term = b[3] if len(b) > 3 else None
        if term in ("s_branch", "s_endpgm", "s_setpc_b64"):
            continue
        if i + 1 < len(blocks):
            b[2].append(blocks[i + 1][0])
    return [(b[0], b[1], b[2]) for b in blocks]


def check_waits_cfg(blocks):
    """check_waits along every control-flow path: each block is replayed
    from every distinct state of outstanding reads that can reach it."""
    by_label = {b[0]: b for b in blocks}
    seen = set()
    bad = set()
    work = [(blocks[0][0], ())]
    while work:
        label, state = work.pop()
        if (label, state) in seen:
            continue
        seen.add((label, state))
        _, insts, succ = by_label[label]
        pending = [set(x) for x in state]
        for ins in insts:
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
                    bad.add((ins, tuple(sorted(busy & regs))))
                pending.append(dst)
            elif op.startswith("s_memtime") or op.startswith("s_load") or op.startswith("s_buffer_load"):
                pending.append(set())
            elif regs & busy:
                bad.add((ins, tuple(sorted(regs & busy))))
            # the 4-bit counter: a wave cannot have more than 15 outstanding
            # (which also bounds the states a loop without waits can reach)
            del pending[:-_LGKM_MAX]
        out = tuple(frozenset(x) for x in pending)
        for nxt in succ:
            if nxt in by_label:
                work.append((nxt, out))
    return sorted(bad)


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
    blocks = _blocks(text, kernel)
    assert any(len(b[2]) > 1 for b in blocks)  # the loop and its branches were found
    bad = check_waits_cfg(blocks)
    assert bad == [], bad[:5]


def test_cfg_checker_follows_the_loop_edge():
    """A read issued at the bottom of a loop and used at its top is pending
    only through the back edge, which a replay in program order never sees;
    the CFG replay flags the missing wait and accepts the loop once the wait
    is in place."""
    def kernel(wait):
        return "\n".join(["kern_pingpong_x:", "s_mov_b32 s0, 0", ".LBB0_1:", wait,
                          "v_mfma_f32_16x16x32_bf16 v[0:3], v[10:13], v[20:23], v[0:3]",
                          "ds_read_b128 v[10:13], v1", "s_cbranch_scc1 .LBB0_1", "s_endpgm",
                          ".Lfunc_end0:"])
    text = kernel("s_nop 0")
    assert check_waits(_kernel_lines(text, "kern_pingpong_x")) == []  # invisible in program order
    bad = check_waits_cfg(_blocks(text, "kern_pingpong_x"))
    assert [b for b in bad if b[0].startswith("v_mfma")]
    assert check_waits_cfg(_blocks(kernel("s_waitcnt lgkmcnt(0)"), "kern_pingpong_x")) == []
