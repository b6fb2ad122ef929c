"""Static check of generated gfx950 assembly: no instruction may read or
write a VGPR/AGPR while a vector-memory load into it is still outstanding.

The decode kernels issue their K loads as inline assembly and wait for them
with explicit `s_waitcnt vmcnt(N)`, so the compiler does not track them.  If
it ever copies, spills or moves such a register before the covering wait,
the copy reads whatever the register held before the data arrived.  This
module finds such accesses by a forward data-flow pass over each kernel's
control-flow graph (basic blocks joined by fall-through, branches and loop
back-edges), iterated to a fixed point.

Model (the gfx9 vector memory counter): every vector memory instruction
(global_, buffer_, scratch_, flat_) increments vmcnt and completes in issue
order; `s_waitcnt vmcnt(N)` returns once at most N of them are outstanding,
i.e. all but the newest N have completed.  The load state at a point is the
list of outstanding instructions, oldest first, each with the set of
registers it writes (empty for stores and for loads into LDS).

Paths.  The compiler often steers control through a 64-bit scalar flag
(`s_mov_b64 s[4:5], -1` on one path, `0` on the other, later
`s_andn2_b64 vcc, exec, s[4:5]` and a branch on vcc), so a branch can be
decided by which path reached it.  The pass therefore keeps, per block, a
small set of path states, each a load state plus the 64-bit scalar flags
known to hold 0 or -1 on that path, and sends a state only along the
branches its flags allow (exec is taken as non-zero: with exec zero no
vector instruction writes or reads a register).  Past a bound on the states
per block, states with the same flags are joined: the load states are
aligned at their newest entries and their entries united position by
position (both a load and a wait act on the newest end, so the joined state
holds exactly the registers some path may still be loading into).
"""
from __future__ import annotations

import re
from dataclasses import dataclass, field

_REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)(?!\w))")
_SPAIR = re.compile(r"\bs\[(\d+):(\d+)\]")
_SREG = re.compile(r"\bs(\d+)\b")
_LABEL = re.compile(r"^(\.?[A-Za-z_][\w.$]*):")
_VMCNT = re.compile(r"vmcnt\((\d+)\)")
_VMEM = ("global_", "buffer_", "scratch_", "flat_")
_MAX_OUT = 64
_MAX_STATES = 16
_ENDS = ("s_endpgm", "s_setpc_b64", "s_trap")
# scalar instructions whose first operand is not written
_NO_SDEST = ("s_cmp", "s_bitcmp", "s_cbranch", "s_branch", "s_waitcnt", "s_nop", "s_barrier", "s_sleep",
             "s_store", "s_endpgm", "s_setprio", "s_sendmsg", "s_dcache", "s_icache", "s_trap", "s_setpc")


def regs_of(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            out.update((kind, r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _sregs_of(text: str) -> set:
    out = set()
    for m in _SPAIR.finditer(text):
        out.update(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in _SREG.finditer(text):
        out.add(int(m.group(1)))
    return out


@dataclass
class Insn:
    index: int
    op: str
    text: str
    # parsed once
    wait: int = -1                 # vmcnt(N) of an s_waitcnt, else -1
    vmem: bool = False
    dest: frozenset = frozenset()  # registers a load writes
    used: frozenset = frozenset()  # registers otherwise accessed
    sdef: frozenset = frozenset()  # scalar registers possibly written
    flag_set: tuple = ()           # (lo, value) for s_mov_b64 s[lo:lo+1], 0 / -1
    vcc_from: tuple = ()           # (lo, negate) for s_and(n2)_b64 vcc, exec, s[lo:lo+1]

    def __post_init__(self):
        op, text = self.op, self.text
        if op == "s_waitcnt":
            m = _VMCNT.search(text)
            self.wait = int(m.group(1)) if m else -1
            return
        ops = _split_operands(text, op)
        if op.startswith(_VMEM):
            self.vmem = True
            dest = regs_of(ops[0]) if (_is_load_with_dest(op) and ops) else set()
            used = set()
            for o in (ops[1:] if dest else ops):
                used |= regs_of(o)
            self.dest, self.used = frozenset(dest), frozenset(used)
        else:
            self.used = frozenset(regs_of(text[len(op):]))
        if ops and not op.startswith(_NO_SDEST):
            if op.startswith("s_") or op.startswith("v_"):
                self.sdef = frozenset(_sregs_of(ops[0]) | (_sregs_of(ops[1]) if op.startswith("v_") and len(ops) > 1
                                                           else set()))
        m = re.match(r"s_mov_b64 s\[(\d+):\d+\], (0|-1)$", text)
        if m:
            self.flag_set = (int(m.group(1)), int(m.group(2)))
        m = re.match(r"s_(and|andn2)_b64 vcc, exec, s\[(\d+):\d+\]$", text)
        if m:
            self.vcc_from = (int(m.group(2)), m.group(1) == "andn2")


def _split_operands(text: str, op: str) -> list:
    rest = text[len(op):].strip()
    return [t.strip() for t in rest.split(",")] if rest else []


def _is_load_with_dest(op: str) -> bool:
    if not op.startswith(_VMEM):
        return False
    if "_lds_" in op or op.endswith("_lds"):
        return False
    return "load" in op


def _key(kind_reg):
    return kind_reg


def _step(state: tuple, ins: Insn, hits: list | None) -> tuple:
    """Load state after `ins`; appends (index, text, registers, load
    indices) to `hits` for an access to a register with an outstanding load."""
    if ins.wait >= 0:
        n = ins.wait
        return state[len(state) - n:] if 0 < n < len(state) else (() if n == 0 else state)
    if ins.used and hits is not None:
        hit, origins = set(), set()
        for regs, origin in state:
            common = regs & ins.used
            if common:
                hit |= common
                origins.add(origin)
        if hit:
            hits.append((ins.index, ins.text, sorted(hit), sorted(origins)))
    if ins.vmem:
        return (state + ((ins.dest, ins.index),))[-_MAX_OUT:]
    return state


def join(a: tuple, b: tuple) -> tuple:
    """Join of two load states, aligned at their newest entries."""
    n = max(len(a), len(b))
    out = []
    for k in range(n, 0, -1):  # k-th newest
        ra, oa = a[-k] if k <= len(a) else (frozenset(), None)
        rb, ob = b[-k] if k <= len(b) else (frozenset(), None)
        out.append((ra | rb, oa if oa is not None else ob))
    return tuple(out)


@dataclass
class Block:
    label: str | None
    insns: list
    succ: list = field(default_factory=list)
    taken: int | None = None   # branch target of a conditional branch
    fall: int | None = None    # fall-through of a conditional branch


def parse_blocks(body: str) -> list:
    """Basic blocks of one function body in layout order, with successors
    (block indices): fall-through, branch targets, nothing after an end."""
    blocks, labels = [], {}
    cur = Block(None, [])
    n = 0

    def close():
        nonlocal cur
        if cur.insns or cur.label is not None:
            blocks.append(cur)
        cur = Block(None, [])

    for raw in body.splitlines():
        line = raw.split(";")[0].strip()
        if not line:
            continue
        m = _LABEL.match(line)
        if m:
            close()
            cur.label = m.group(1)
            labels[m.group(1)] = len(blocks)
            continue
        if line.startswith("."):
            continue  # directives
        op = line.split()[0]
        cur.insns.append(Insn(n, op, line))
        n += 1
        if op.startswith(("s_branch", "s_cbranch")) or op in _ENDS:
            close()
    close()
    for i, b in enumerate(blocks):
        last = b.insns[-1] if b.insns else None
        nxt = [i + 1] if i + 1 < len(blocks) else []
        if last is None:
            b.succ = nxt
        elif last.op == "s_branch":
            b.succ = [labels[last.text.split()[-1]]]
        elif last.op.startswith("s_cbranch"):
            tgt = last.text.split()[-1]
            b.taken = labels.get(tgt)
            b.fall = i + 1 if i + 1 < len(blocks) else None
            b.succ = ([b.taken] if b.taken is not None else []) + nxt
        elif last.op in _ENDS:
            b.succ = []
        else:
            b.succ = nxt
    return blocks


def _run_block(b: Block, state: tuple, flags: frozenset, hits):
    """Load state and flags at the block's end, and the successors the path
    can take."""
    fl = dict(flags)
    vcc = None  # None unknown; True non-zero; False zero
    for ins in b.insns:
        state = _step(state, ins, hits)
        if ins.vcc_from:
            lo, neg = ins.vcc_from
            v = fl.get(lo)
            vcc = None if v is None else ((v == 0) if neg else (v == -1))
        elif "vcc" in ins.text and not ins.op.startswith("s_cbranch"):
            vcc = None
        if ins.flag_set:
            fl[ins.flag_set[0]] = ins.flag_set[1]
        elif ins.sdef:
            for lo in list(fl):
                if lo in ins.sdef or lo + 1 in ins.sdef:
                    del fl[lo]
    succ = b.succ
    last = b.insns[-1] if b.insns else None
    if last is not None and last.op in ("s_cbranch_vccz", "s_cbranch_vccnz") and vcc is not None:
        take = (not vcc) if last.op == "s_cbranch_vccz" else vcc
        nxt = b.taken if take else b.fall
        succ = [nxt] if nxt is not None else []
    return state, frozenset(fl.items()), succ


def _meet(f1: frozenset, f2: frozenset) -> frozenset:
    """Flags known on both paths (same value)."""
    return f1 & f2


def _add(states: dict, i: int, st: tuple, fl: frozenset) -> bool:
    """Add a path state to block i; returns whether the block's set grew.

    The set is kept to _MAX_STATES entries: first states with equal load
    states are merged (keeping the flags both know), then states with equal
    flags (joining their load states), then all of them."""
    cur = states.setdefault(i, {})
    if fl in cur:
        new = join(cur[fl], st)
        if new == cur[fl]:
            return False
        cur[fl] = new
        return True
    before = dict(cur)
    cur[fl] = st
    if len(cur) > _MAX_STATES:
        by_loads = {}
        for f, s2 in cur.items():
            by_loads[s2] = _meet(by_loads[s2], f) if s2 in by_loads else f
        merged = {}
        for s2, f in by_loads.items():
            merged[f] = join(merged[f], s2) if f in merged else s2
        if len(merged) > _MAX_STATES:
            allf, alls = None, ()
            for f, s2 in merged.items():
                allf = f if allf is None else _meet(allf, f)
                alls = join(alls, s2)
            merged = {allf: alls}
        states[i] = merged
        cur = merged
    return cur != before


def scan_function(body: str) -> list:
    """(instruction index, text, registers, indices of the loads) of every
    access to a register that some path may still be loading into, from a
    fixed point of the forward data flow over the control-flow graph."""
    blocks = parse_blocks(body)
    if not blocks:
        return []
    states = {}
    _add(states, 0, (), frozenset())
    work, queued = [0], {0}
    while work:
        i = work.pop()
        queued.discard(i)
        for fl, st in list(states[i].items()):
            out, fl2, succ = _run_block(blocks[i], st, fl, None)
            for s in succ:
                if _add(states, s, out, fl2) and s not in queued:
                    work.append(s)
                    queued.add(s)
    hits = []
    seen = set()
    for i in sorted(states):
        for fl, st in states[i].items():
            h = []
            _run_block(blocks[i], st, fl, h)
            for x in h:
                if x[0] not in seen:
                    seen.add(x[0])
                    hits.append((x[0], x[1], [r for r in x[2]], x[3]))
    hits.sort()
    return hits


def kernel_bodies(asm: str, prefix: str) -> dict:
    """Function name -> body for every function whose name starts with
    `prefix` (mangled)."""
    out = {}
    for m in re.finditer(r"\n(" + re.escape(prefix) + r"\w*):[^\n]*\n(.*?)\n\.Lfunc_end", asm, re.S):
        out[m.group(1)] = m.group(2)
    return out
