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


def _scalar_effect(op: str, text: str, ops: list) -> tuple:
    """What an instruction does to the scalar facts tracked on a path:
    ("cmp",) a comparison (a new SCC symbol); ("csel", lo, a, b); ("mov64",
    lo, src_lo or None, const); ("mov32", dst, src or None, const); ("xor1",
    dst_lo, src_lo); ("vcc", lo, negate); ("wlane", vgpr, sreg, lane);
    ("rlane", sreg, vgpr, lane); ("vccmov", src_lo or None, const); ("vccself", negate); else ("other", clobbers_scc, clobbers_vcc,
    vgpr written or -1)."""
    if re.match(r"^s_(?:cmp|bitcmp)", op):
        return ("cmp",)
    m = re.match(r"^s_cselect_b64 s\[(\d+):\d+\], (-1|0), (-1|0)$", text)
    if m:
        return ("csel", int(m.group(1)), int(m.group(2)), int(m.group(3)))
    m = re.match(r"^s_mov_b64 s\[(\d+):\d+\], (?:s\[(\d+):\d+\]|(-1|0))$", text)
    if m:
        return ("mov64", int(m.group(1)), None if m.group(2) is None else int(m.group(2)),
                None if m.group(3) is None else int(m.group(3)))
    m = re.match(r"^s_mov_b64 vcc, (?:s\[(\d+):\d+\]|(-1|0))$", text)
    if m:
        return ("vccmov", None if m.group(1) is None else int(m.group(1)),
                None if m.group(2) is None else int(m.group(2)))
    m = re.match(r"^s_mov_b32 s(\d+), (?:s(\d+)|(-1|0))$", text)
    if m:
        return ("mov32", int(m.group(1)), None if m.group(2) is None else int(m.group(2)),
                None if m.group(3) is None else int(m.group(3)))
    m = re.match(r"^s_xor_b64 s\[(\d+):\d+\], s\[(\d+):\d+\], -1$", text)
    if m:
        return ("xor1", int(m.group(1)), int(m.group(2)))
    m = re.match(r"^s_(and|andn2)_b64 vcc, exec, s\[(\d+):\d+\]$", text)
    if m:
        return ("vcc", int(m.group(2)), m.group(1) == "andn2")
    # the same on vcc itself (a branch on a flag the compiler already folded
    # into vcc); exec is taken as non-zero, as on any path where a lane runs
    m = re.match(r"^s_(and|andn2)_b64 vcc, exec, vcc$", text)
    if m:
        return ("vccself", m.group(1) == "andn2")
    m = re.match(r"^v_writelane_b32 v(\d+), s(\d+), (\d+)$", text)
    if m:
        return ("wlane", int(m.group(1)), int(m.group(2)), int(m.group(3)))
    m = re.match(r"^v_readlane_b32 s(\d+), v(\d+), (\d+)$", text)
    if m:
        return ("rlane", int(m.group(1)), int(m.group(2)), int(m.group(3)))
    clob_scc = op.startswith("s_") and not op.startswith(("s_cbranch", "s_branch", "s_waitcnt", "s_nop", "s_sleep",
                                                           "s_barrier", "s_setprio", "s_load", "s_store",
                                                           "s_mov", "s_cselect"))
    clob_vcc = "vcc" in text and not op.startswith("s_cbranch")
    vdef = -1
    if op.startswith("v_") and not op.startswith(("v_readlane", "v_readfirstlane", "v_cmp")) and ops:
        regs = [r for k, r in regs_of(ops[0]) if k == "v"]
        vdef = regs[0] if len(regs) == 1 else (-2 if regs else -1)
    return ("other", clob_scc, clob_vcc, vdef)


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
    sc: tuple = ()                 # its effect on the scalar facts (see _scalar_effect)

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
        self.sc = _scalar_effect(op, text, ops)


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


# Scalar facts on a path.  A value is ("k", 0 or -1), a known 64-bit flag
# (one half of it for a 32-bit register), or ("s", id, negated), the
# boolean a comparison produced (id: the comparison's instruction index).
# `env` maps scalar registers and VGPR-lane spill slots ("l", vgpr, lane) to
# values, and "scc"/"vcc" to the condition bits; `known` maps comparison
# ids to the outcome a branch on this path has fixed.
def _neg(v):
    if v is None:
        return None
    if v[0] == "k":
        return ("k", -1 if v[1] == 0 else 0)
    return ("s", v[1], not v[2])


def _truth(v, known):
    """True/False if the flag's value is fixed on this path, else None."""
    if v is None:
        return None
    if v[0] == "k":
        return v[1] == -1
    t = known.get(v[1])
    return None if t is None else (t != v[2])


def _pair(env, lo):
    a, b = env.get(lo), env.get(lo + 1)
    return a if a == b else None


def _run_block(b: Block, state: tuple, flags, hits):
    """Load state and scalar facts at the block's end, and the successors
    the path can take (with the facts each branch adds)."""
    env = dict(flags[0]) if flags else {}
    known = dict(flags[1]) if flags else {}
    for ins in b.insns:
        state = _step(state, ins, hits)
        e = ins.sc
        k = e[0] if e else "other"
        if k == "cmp":
            env["scc"] = ("s", ins.index, False)
            known.pop(ins.index, None)  # a new outcome each time it runs
        elif k == "csel":
            lo, a, bb = e[1], e[2], e[3]
            sc = env.get("scc")
            v = ("k", a) if a == bb else (None if sc is None else (sc if a == -1 else _neg(sc)))
            env[lo] = env[lo + 1] = v
        elif k == "mov64":
            v = ("k", e[3]) if e[3] is not None else _pair(env, e[2])
            env[e[1]] = env[e[1] + 1] = v
        elif k == "mov32":
            env[e[1]] = ("k", e[3]) if e[3] is not None else env.get(e[2])
        elif k == "xor1":
            v = _neg(_pair(env, e[2]))
            env[e[1]] = env[e[1] + 1] = v
            env["scc"] = None
        elif k == "vcc":
            v = _pair(env, e[1])
            env["vcc"] = _neg(v) if e[2] else v
            env["scc"] = None
        elif k == "vccmov":
            env["vcc"] = ("k", e[2]) if e[2] is not None else _pair(env, e[1])
        elif k == "vccself":
            v = env.get("vcc")
            env["vcc"] = _neg(v) if e[1] else v
            env["scc"] = None
        elif k == "wlane":
            env[("l", e[1], e[3])] = env.get(e[2])
        elif k == "rlane":
            env[e[1]] = env.get(("l", e[2], e[3]))
        else:
            if e and e[1]:
                env["scc"] = None
            if e and e[2]:
                env["vcc"] = None
            for r in ins.sdef:
                env.pop(r, None)
            if e and e[3] != -1:
                dead = [key for key in env if type(key) is tuple and (e[3] == -2 or key[1] == e[3])]
                for key in dead:
                    del env[key]
    out = []
    last = b.insns[-1] if b.insns else None
    cond = None
    if last is not None and last.op in ("s_cbranch_vccz", "s_cbranch_vccnz"):
        cond, nz = env.get("vcc"), last.op == "s_cbranch_vccnz"
    elif last is not None and last.op in ("s_cbranch_scc0", "s_cbranch_scc1"):
        cond, nz = env.get("scc"), last.op == "s_cbranch_scc1"
    envf = frozenset((kk, vv) for kk, vv in env.items() if vv is not None)
    if cond is not None and b.taken is not None:
        tv = _truth(cond, known)
        for succ, take in ((b.taken, True), (b.fall, False)):
            if succ is None:
                continue
            want = take if nz else not take  # the value of cond on this edge
            if tv is not None and tv != want:
                continue
            k2 = dict(known)
            if cond[0] == "s":
                k2[cond[1]] = want != cond[2]
            out.append((succ, (envf, frozenset(k2.items()))))
    else:
        kf = frozenset(known.items())
        out = [(s2, (envf, kf)) for s2 in b.succ]
    return state, out


def _meet(f1, f2):
    """Facts both paths share."""
    if not f1 or not f2:
        return (frozenset(), frozenset())
    return (f1[0] & f2[0], f1[1] & f2[1])


def _add(states: dict, i: int, st: tuple, fl) -> bool:
    """Add a path state to block i; returns whether the block's set grew.
    Past _MAX_STATES distinct facts the block keeps one state: the facts
    all paths share and the join of their load states (monotone, so the
    iteration ends)."""
    cur = states.setdefault(i, {})
    if fl in cur:
        new = join(cur[fl], st)
        if new == cur[fl]:
            return False
        cur[fl] = new
        return True
    # covered by a state that knows less and may be loading at least as much
    for f2, s2 in cur.items():
        if f2[0] <= fl[0] and f2[1] <= fl[1] and join(s2, st) == s2:
            return False
    if len(cur) + 1 > _MAX_STATES:
        allf, alls = fl, st
        for f, s2 in cur.items():
            allf = _meet(allf, f)
            alls = join(alls, s2)
        if len(cur) == 1 and allf in cur and cur[allf] == alls:
            return False
        states[i] = {allf: alls}
        return True
    cur[fl] = st
    return True


def scan_function(body: str) -> list:
    """(instruction index, text, registers, indices of the loads) of every
    access to a register that some path may still be loading into, from a
    fixed point of the forward data flow over the control-flow graph."""
    blocks = parse_blocks(body)
    if not blocks:
        return []
    states = {}
    _add(states, 0, (), ())
    work, queued = [0], {0}
    while work:
        i = work.pop()
        queued.discard(i)
        for fl, st in list(states[i].items()):
            out, succ = _run_block(blocks[i], st, fl, None)
            for s, fl2 in succ:
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
