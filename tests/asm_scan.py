"""Static check of generated gfx950 assembly: no instruction may read or
write a VGPR/AGPR while a vector-memory load into it is still outstanding.

The decode kernels issue their K loads as inline assembly and wait for them
with explicit `s_waitcnt vmcnt(N)`, so the compiler does not track them.  If
it ever copies, spills or moves such a register before the covering wait,
the copy reads whatever the register held before the data arrived.  This
module finds such accesses by a forward data-flow pass over each kernel's
instructions in layout order (see scan_function for its limits).

Model (the gfx9 vector memory counter): every vector memory instruction
(global_, buffer_, scratch_, flat_) increments vmcnt and completes in issue
order; `s_waitcnt vmcnt(N)` returns once at most N of them are outstanding,
i.e. all but the newest N have completed.  The state at a point is the list
of outstanding instructions, oldest first, each as the set of registers it
writes (empty for stores and for loads into LDS).
"""
from __future__ import annotations

import re
from dataclasses import dataclass

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
_LABEL = re.compile(r"^(\.?[A-Za-z_][\w.$]*):")
_VMCNT = re.compile(r"vmcnt\((\d+)\)")
_VMEM = ("global_", "buffer_", "scratch_", "flat_")
_MAX_OUT = 64


def regs_of(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            out.update((kind, r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


@dataclass
class Insn:
    index: int
    op: str
    text: str


def _split_operands(text: str, op: str) -> list:
    rest = text[len(op):].strip()
    return [t.strip() for t in rest.split(",")] if rest else []


def _is_load_with_dest(op: str) -> bool:
    if not op.startswith(_VMEM):
        return False
    if "_lds_" in op or op.endswith("_lds"):
        return False
    return "load" in op


def _step(state: tuple, ins: Insn, hits: list | None) -> tuple:
    if ins.op == "s_waitcnt":
        m = _VMCNT.search(ins.text)
        if m:
            n = int(m.group(1))
            state = state[len(state) - n:] if 0 < n < len(state) else (() if n == 0 else state)
        return state
    pending = {}
    for entry in state:
        for kind, reg, origin in entry:
            pending.setdefault((kind, reg), set()).add(origin)
    ops = _split_operands(ins.text, ins.op)
    if ins.op.startswith(_VMEM):
        dest = regs_of(ops[0]) if (_is_load_with_dest(ins.op) and ops) else set()
        used = set()
        for o in (ops[1:] if dest else ops):
            used |= regs_of(o)
    else:
        dest, used = set(), regs_of(ins.text[len(ins.op):])
    # a load may overwrite the target of an older outstanding load (they
    # complete in order); any other access to such a register is a hazard
    hit = sorted(r for r in used if r in pending)
    if hits is not None and hit:
        origins = sorted(set().union(*(pending[r] for r in hit)))
        hits.append((ins.index, ins.text, hit, origins))
    if ins.op.startswith(_VMEM):
        state = state + (frozenset((k, r, ins.index) for k, r in dest),)
        return state[-_MAX_OUT:]
    return state


def scan_function(body: str) -> list:
    """(instruction index, text, registers, indices of the loads) of every
    access to a register with an outstanding load into it, in layout order.

    The scan follows the instructions as laid out.  At a label reached only
    by a jump (the instruction before it ends the path: an unconditional
    branch or the end of the program) the incoming state is unknown and is
    taken as empty, so a hazard across such a jump is not seen; everything a
    wave executes between a load and the wait that covers it within one
    layout-contiguous stretch is."""
    state, hits, prev = (), [], None
    for ins in parse_function_linear(body):
        if ins is None:  # label
            if prev is not None and prev.op.startswith(("s_branch", "s_endpgm", "s_setpc")):
                state = ()
            continue
        state = _step(state, ins, hits)
        prev = ins
    return hits


def parse_function_linear(body: str) -> list:
    """Instructions of one function body in layout order, with None at each
    label."""
    out = []
    for raw in body.splitlines():
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if _LABEL.match(line):
            out.append(None)
            continue
        if line.startswith("."):
            continue  # directives
        out.append(Insn(len(out), line.split()[0], line))
    return out


def kernel_bodies(asm: str, prefix: str) -> dict:
    """Function name -> body for every function whose name starts with
    `prefix` (mangled)."""
    out = {}
    for m in re.finditer(r"\n(" + re.escape(prefix) + r"\w*):[^\n]*\n(.*?)\n\.Lfunc_end", asm, re.S):
        out[m.group(1)] = m.group(2)
    return out
