"""Static check of the kernels' gfx950 assembly: no instruction may read or overwrite a
register that an LDS read still in flight is going to write.

The hand-scheduled kernels issue their LDS reads as inline assembly and tie the results to
an explicit ``s_waitcnt lgkmcnt(N)``; the compiler does not know those reads complete
asynchronously, so nothing but this check stops it from copying a result (or reusing its
register) before the wait, for instance where two paths that issue different reads join.

Hardware rules followed (gfx9 family):

* LDS operations complete in issue order; ``lgkmcnt(N)`` returns once at most N operations
  counted by that counter are outstanding, so every LDS operation but the N most recent is
  complete after it.
* Scalar-memory loads share the counter but may complete out of order, so only
  ``lgkmcnt(0)`` is taken to complete them.

The check is a forward data-flow analysis over the control-flow graph of each function
(basic blocks split at labels and after branches; a conditional branch continues both at
its target and at the next instruction). The state at a point is the list of possibly
pending LDS destinations, oldest first, and the set of possibly pending scalar-load
destinations. Where paths join, the lists are aligned at their most recent end and merged
entry by entry (a union), and the scalar sets are merged: a register counts as pending if
it may be pending on any path reaching the point. The states only grow, so iterating to a
fixed point ends.
"""
from __future__ import annotations

import re
import sys
from typing import Dict, FrozenSet, List, Optional, Set, Tuple

Reg = Tuple[str, int]
State = Tuple[Tuple[FrozenSet[Reg], ...], FrozenSet[Reg]]

_LGKM_MAX = 15       # gfx9: a 4-bit counter, so at most 15 operations are outstanding


def _regs(tok: str) -> Set[Reg]:
    tok = tok.strip().split()[0] if tok.strip() else ""
    m = re.match(r"([vas])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([vas])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _lgkm_wait(s: str) -> Optional[int]:
    """The lgkmcnt limit of an s_waitcnt, or None if it does not constrain that counter."""
    m = re.search(r"lgkmcnt\((\d+)\)", s)
    if m:
        return int(m.group(1))
    m = re.match(r"s_waitcnt\s+(0x[0-9a-fA-F]+|\d+)\s*$", s)
    if m:
        v = int(m.group(1), 0)
        n = (v >> 8) & 0xF
        return None if n == _LGKM_MAX else n
    return None


class _Insn:
    __slots__ = ("line", "text", "op", "args")

    def __init__(self, line: int, text: str):
        self.line, self.text = line, text
        self.op = text.split()[0]
        self.args = text[len(self.op):].split(",")


def _parse(asm_text: str):
    """Instructions and labels of the text, in order. Returns (insns, label -> index of the
    next instruction, indices where a function begins)."""
    insns: List[_Insn] = []
    labels: Dict[str, int] = {}
    entries: List[int] = []
    for ln, line in enumerate(asm_text.splitlines(), 1):
        s = line.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":"):
            name = s[:-1]
            labels[name] = len(insns)
            if not name.startswith("."):
                entries.append(len(insns))
            continue
        if s.startswith("."):
            continue
        insns.append(_Insn(ln, s))
    return insns, labels, entries


def _successors(i: int, ins: _Insn, labels: Dict[str, int], n: int) -> List[int]:
    op = ins.op
    if op in ("s_endpgm", "s_setpc_b64", "s_trap"):
        return []
    target = None
    if op.startswith("s_branch") or op.startswith("s_cbranch"):
        name = ins.args[0].strip().split()[0] if ins.args and ins.args[0].strip() else ""
        target = labels.get(name)
    if op == "s_branch":
        return [target] if target is not None else []
    out = [i + 1] if i + 1 < n else []
    if target is not None:
        out.append(target)
    return out


def _join(a: Optional[State], b: State) -> State:
    if a is None:
        return b
    la, lb = a[0], b[0]
    n = max(len(la), len(lb))
    pa = (frozenset(),) * (n - len(la)) + la
    pb = (frozenset(),) * (n - len(lb)) + lb
    return tuple(x | y for x, y in zip(pa, pb)), a[1] | b[1]


def _step(ins: _Insn, st: State, out: List[str]) -> State:
    lds, smem = st
    s, op = ins.text, ins.op
    if op == "s_waitcnt":
        n = _lgkm_wait(s)
        if n is None:
            return st
        return (lds[len(lds) - n:] if n else ()), (smem if n else frozenset())
    live = set(smem).union(*lds) if lds else set(smem)
    args = ins.args
    if op.startswith(("ds_read", "ds_write", "ds_load", "ds_store", "ds_bpermute",
                      "ds_permute", "ds_swizzle", "ds_add", "ds_append", "ds_consume")):
        writes_reg = op.startswith(("ds_read", "ds_load", "ds_bpermute", "ds_permute",
                                    "ds_swizzle")) or "_rtn" in op
        srcs = set().union(*[_regs(a) for a in (args[1:] if writes_reg else args)])
        dst = _regs(args[0]) if writes_reg else set()
        if (srcs | dst) & live:
            out.append(f"line {ins.line}: {s}")
        lds = (lds + (frozenset(dst),))[-_LGKM_MAX:]
        return lds, smem
    if op.startswith(("s_load", "s_buffer_load")):
        dst = _regs(args[0])
        srcs = set().union(*[_regs(a) for a in args[1:]])
        if (srcs | dst) & live:
            out.append(f"line {ins.line}: {s}")
        return lds, smem | frozenset(dst)
    if set().union(*[_regs(a) for a in args]) & live:
        out.append(f"line {ins.line}: {s}")
    return st


def violations(asm_text: str) -> List[str]:
    insns, labels, entries = _parse(asm_text)
    n = len(insns)
    if n == 0:
        return []
    state: List[Optional[State]] = [None] * n
    empty: State = ((), frozenset())
    for e in (entries or [0]):
        if e < n:
            state[e] = empty
    work = [e for e in (entries or [0]) if e < n]
    while work:
        i = work.pop()
        sink: List[str] = []
        nxt = _step(insns[i], state[i], sink)
        for j in _successors(i, insns[i], labels, n):
            merged = _join(state[j], nxt)
            if merged != state[j]:
                state[j] = merged
                work.append(j)
    found: List[str] = []
    for i in range(n):
        if state[i] is not None:
            _step(insns[i], state[i], found)
    return found


def main(paths: List[str]) -> int:
    bad = 0
    for p in paths:
        v = violations(open(p).read())
        for line in v[:20]:
            print(f"{p}: {line}")
        print(f"{p}: {len(v)} violations")
        bad += len(v)
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
