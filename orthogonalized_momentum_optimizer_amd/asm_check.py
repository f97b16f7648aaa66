"""Static check of the kernels' gfx950 assembly: no instruction may read or overwrite a
register that an LDS read still in flight is going to write.

The hand-scheduled kernels issue their LDS reads as inline assembly and tie the results to
an explicit ``s_waitcnt lgkmcnt(0)``; the compiler does not know those reads complete
asynchronously, so nothing but this check stops it from copying a result (or reusing its
register) before the wait. The check follows the hardware rule: LDS operations complete in
order, and ``lgkmcnt(N)`` returns once at most the N most recent LDS or scalar-memory
operations are outstanding. It walks straight-line code and forgets pending reads at every
label, so a read that reaches a use only through a branch is not followed.
"""
from __future__ import annotations

import re
import sys
from typing import List, Set, Tuple

Reg = Tuple[str, int]


def _regs(tok: str) -> Set[Reg]:
    tok = tok.strip().split()[0] if tok.strip() else ""
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def violations(asm_text: str) -> List[str]:
    out: List[str] = []
    pending: List[Set[Reg]] = []  # destinations of outstanding LDS/scalar-memory operations
    for ln, line in enumerate(asm_text.splitlines(), 1):
        s = line.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":"):
            pending = []
            continue
        if s.startswith("."):
            continue
        op = s.split()[0]
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", s)
            if m:
                n = int(m.group(1))
                pending = pending[len(pending) - n:] if n else []
            continue
        args = s[len(op):].split(",")
        live = set().union(*pending) if pending else set()
        if op.startswith(("ds_read", "ds_write", "s_load", "s_buffer_load")):
            is_read = op.startswith("ds_read")
            srcs = set().union(*[_regs(a) for a in (args[1:] if is_read else args)])
            dst = _regs(args[0]) if is_read else set()
            if (srcs | dst) & live:
                out.append(f"line {ln}: {s}")
            pending.append(dst)
            continue
        if set().union(*[_regs(a) for a in args]) & live:
            out.append(f"line {ln}: {s}")
    return out


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
