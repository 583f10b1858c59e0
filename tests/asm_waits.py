"""Static check of the kernels' inline-asm LDS reads in their gfx950 assembly.

The kernels issue their LDS reads as inline asm (`ds_read_b128`,
`ds_read_b64_tr_b16`, ...) and wait for them with explicit
`s_waitcnt lgkmcnt(n)`: the compiler sees neither the reads' latency nor
their count.  LDS reads complete in the order they were issued, so after
`s_waitcnt lgkmcnt(n)` all but the last n outstanding reads have written
their registers.  This module walks a kernel's assembly in program order,
keeps the queue of outstanding reads with their destination registers, and
reports every instruction that reads or writes a register that an
outstanding read has yet to write (a missing or too loose wait), or that
uses a pending register as an LDS address.

The walk is straight-line (labels and branches are not followed); the
kernels wait for every read before their barriers and loop heads, so no
read is outstanding across a branch.  Scalar loads also count in lgkmcnt
and can complete out of order; they only make a wait stricter and are not
tracked.

The kernels' matrix products are inline asm too, so the compiler does not
space other instructions from them either; the kernels do it with s_nop.
Two more walks check that spacing against what the compiler keeps for its
own gfx950 MFMAs (read off its output): at least 12 wait states between an
MFMA and any non-MFMA instruction that reads or writes its result, or an
MFMA that takes it as a multiplicand (a product accumulating into it needs
none), and at least 2 between a vector instruction and an MFMA that reads
the register it wrote.  A wait state is one instruction, or n + 1 for
s_nop n; an MFMA in between counts as one, which understates the time it
takes, so the walks err on the strict side.
"""
from __future__ import annotations

import re

_RANGE = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")


def _regs(tok: str) -> set:
    out = set()
    for m in _RANGE.finditer(tok):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            out.update((m.group(3), r) for r in range(int(m.group(4)), int(m.group(5)) + 1))
    return out


def kernel_lines(asm: str, symbol: str) -> list:
    a = asm.index(symbol + ":")
    b = asm.index(".Lfunc_end", a)
    return asm[a:b].splitlines()


def check(lines: list) -> tuple:
    """Returns (LDS reads, lgkmcnt waits, list of violations)."""
    queue, bad, nreads, nwaits = [], [], 0, 0
    for i, line in enumerate(lines):
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        op = t.split()[0]
        rest = t[len(op):].strip()
        ops = [x.strip() for x in rest.split(",")] if rest else []
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", t)
            if m:
                nwaits += 1
                n = int(m.group(1))
                while len(queue) > n:
                    queue.pop(0)
            continue
        used = set().union(*(_regs(x) for x in ops)) if ops else set()
        if op.startswith("ds_read"):
            dest = _regs(ops[0])
            addr = set().union(*(_regs(x) for x in ops[1:])) if len(ops) > 1 else set()
            for pend in queue:
                if addr & pend:
                    bad.append((i, "address of a pending read", t))
                if dest & pend:
                    bad.append((i, "overwrites a pending read", t))
            queue.append(dest)
            nreads += 1
            continue
        for pend in queue:
            if used & pend:
                bad.append((i, "uses a pending read", t))
                break
    return nreads, nwaits, bad


def _walk(lines):
    """(line index, opcode, operand list, text) of every instruction."""
    for i, line in enumerate(lines):
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        op = t.split()[0]
        rest = t[len(op):].strip()
        yield i, op, ([x.strip() for x in rest.split(",")] if rest else []), t


def _ws(op, ops):
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def check_mfma_results(lines: list, need: int = 12) -> list:
    """Instructions that touch an MFMA's result fewer than `need` wait
    states after it (an MFMA accumulating into it excepted)."""
    pend, bad = [], []  # (result registers, wait states since, line)
    for i, op, ops, t in _walk(lines):
        if op.startswith("v_mfma"):
            ab = _regs(ops[1]) | _regs(ops[2])
            bad += [(i, w, t) for d, w, _ in pend if ab & d]
        elif op != "s_nop":
            used = set().union(*(_regs(x) for x in ops)) if ops else set()
            bad += [(i, w, t) for d, w, _ in pend if used & d]
        n = _ws(op, ops)
        pend = [(d, w + n, l) for d, w, l in pend if w + n < need]
        if op.startswith("v_mfma"):
            pend.append((_regs(ops[0]), 0, i))
    return bad


def check_mfma_operands(lines: list, need: int = 2) -> list:
    """MFMAs that read a register a vector instruction wrote fewer than
    `need` wait states before."""
    pend, bad = [], []
    for i, op, ops, t in _walk(lines):
        if op.startswith("v_mfma"):
            src = set().union(*(_regs(x) for x in ops[1:4]))
            bad += [(i, w, t) for d, w, _ in pend if src & d]
        n = _ws(op, ops)
        pend = [(d, w + n, l) for d, w, l in pend if w + n < need]
        if (op.startswith("v_") and not op.startswith(("v_mfma", "v_cmp", "v_readlane", "v_readfirstlane"))
                and ops):
            pend.append((_regs(ops[0]), 0, i))
    return bad
