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

The walks follow the branches: the state at a label merges the states of
the fall-through and of every branch to it (a backward branch's on a
further pass over the kernel, until the states stop changing).  A merge
errs on the strict side: of the outstanding reads it keeps the longer
queue, each position (counted from the newest read) with the registers of
every path, and of the products every pending result with its shortest
distance.  Scalar loads also count in lgkmcnt and can complete out of
order; they only make a wait stricter and are not tracked.

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


_LABEL = re.compile(r"^(\.L\w+):")


def _parse(lines):
    """('label', name) or ('inst', line index, opcode, operands, text) items."""
    out = []
    for i, line in enumerate(lines):
        t = line.split(";")[0].strip()
        if not t:
            continue
        m = _LABEL.match(t)
        if m:
            out.append(("label", m.group(1)))
            continue
        if t.startswith(".") or t.endswith(":"):
            continue
        op = t.split()[0]
        rest = t[len(op):].strip()
        out.append(("inst", i, op, [x.strip() for x in rest.split(",")] if rest else [], t))
    return out


def _flow(lines, init, step, merge, passes=40):
    """Runs step(state, i, op, ops, text, bad) over the instructions in
    program order along the branches; returns the violations step reported
    on the last pass.  States are immutable values."""
    items = _parse(lines)
    back = {}
    for _ in range(passes):
        bad, incoming, seen, new_back, state = [], {}, set(), {}, init
        for it in items:
            if it[0] == "label":
                lab = it[1]
                seen.add(lab)
                ins = incoming.pop(lab, [])
                if state is not None:
                    ins.append(state)
                if lab in back:
                    ins.append(back[lab])
                state = merge(ins) if ins else None
                continue
            _, i, op, ops, t = it
            if state is None:  # reached only by a backward branch: known from the pass before
                state = init
            state = step(state, i, op, ops, t, bad)
            if op == "s_branch" or op.startswith("s_cbranch"):
                tgt = ops[0]
                if tgt in seen:
                    new_back[tgt] = merge([new_back[tgt], state]) if tgt in new_back else state
                else:
                    incoming.setdefault(tgt, []).append(state)
                if op == "s_branch":
                    state = None
            elif op == "s_endpgm":
                state = None
        if new_back == back:
            return bad
        back = new_back
    raise AssertionError("branch states did not settle")


_QMAX = 16


def _cap(q):
    """At most _QMAX entries (a loop that never waits grows its queue every
    pass): the oldest entry joins the next one, which retires later."""
    while len(q) > _QMAX:
        q = (q[0] | q[1],) + q[2:]
    return q


def _merge_queues(qs):
    n = max(len(q) for q in qs)
    return _cap(tuple(frozenset().union(*(q[len(q) - n + k] for q in qs if len(q) - n + k >= 0)) for k in range(n)))


def _merge_pending(ps):
    best = {}
    for p in ps:
        for d, w in p:
            best[d] = min(w, best.get(d, w))
    return tuple(sorted(best.items(), key=lambda x: (x[1], sorted(x[0]))))


def check(lines: list) -> tuple:
    """Returns (LDS reads, lgkmcnt waits, list of violations)."""
    count = {"reads": set(), "waits": set()}

    def step(queue, i, op, ops, t, bad):
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", t)
            if m:
                count["waits"].add(i)
                n = int(m.group(1))
                if len(queue) > n:
                    queue = queue[len(queue) - n:]
            return queue
        used = set().union(*(_regs(x) for x in ops)) if ops else set()
        if op.startswith("ds_read"):
            dest = _regs(ops[0])
            addr = set().union(*(_regs(x) for x in ops[1:])) if len(ops) > 1 else set()
            for pend in queue:
                if addr & pend:
                    bad.append((i, "address of a pending read", t))
                if dest & pend:
                    bad.append((i, "overwrites a pending read", t))
            count["reads"].add(i)
            return _cap(queue + (frozenset(dest),))
        for pend in queue:
            if used & pend:
                bad.append((i, "uses a pending read", t))
                break
        return queue

    bad = _flow(lines, (), step, _merge_queues)
    return len(count["reads"]), len(count["waits"]), bad


def _walk(lines):
    """(line index, opcode, operand list, text) of every instruction."""
    for it in _parse(lines):
        if it[0] == "inst":
            yield it[1:]


def _ws(op, ops):
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def check_mfma_results(lines: list, need: int = 12) -> list:
    """Instructions that touch an MFMA's result fewer than `need` wait
    states after it (an MFMA accumulating into it excepted)."""

    def step(pend, i, op, ops, t, bad):
        if op.startswith("v_mfma"):
            ab = _regs(ops[1]) | _regs(ops[2])
            bad += [(i, w, t) for d, w in pend if ab & d]
        elif op != "s_nop":
            used = set().union(*(_regs(x) for x in ops)) if ops else set()
            bad += [(i, w, t) for d, w in pend if used & d]
        n = _ws(op, ops)
        pend = tuple((d, w + n) for d, w in pend if w + n < need)
        if op.startswith("v_mfma"):
            pend = _merge_pending([pend, ((frozenset(_regs(ops[0])), 0),)])
        return pend

    return _flow(lines, (), step, _merge_pending)


def check_mfma_operands(lines: list, need: int = 2) -> list:
    """MFMAs that read a register a vector instruction wrote fewer than
    `need` wait states before."""

    def step(pend, i, op, ops, t, bad):
        if op.startswith("v_mfma"):
            src = set().union(*(_regs(x) for x in ops[1:4]))
            bad += [(i, w, t) for d, w in pend if src & d]
        n = _ws(op, ops)
        pend = tuple((d, w + n) for d, w in pend if w + n < need)
        if (op.startswith("v_") and not op.startswith(("v_mfma", "v_cmp", "v_readlane", "v_readfirstlane"))
                and ops):
            pend = _merge_pending([pend, ((frozenset(_regs(ops[0])), 0),)])
        return pend

    return _flow(lines, (), step, _merge_pending)
