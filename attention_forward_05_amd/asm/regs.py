"""Register allocation, instruction emission and hazard tracking for the
gfx950 attention kernel generator.

The kernel is written with explicit registers.  `Emitter` keeps the text and
a small model of the hazards the hardware leaves to software, inserting the
s_nop / s_waitcnt each instruction needs:

* an MFMA result read (or overwritten) by a non-MFMA instruction: 12 wait
  states after the MFMA issues;
* a VALU result read by an MFMA (any operand): 2 wait states;
* a VALU result read by v_permlane32_swap: 2 wait states;
* a VALU result read by v_readfirstlane / v_readlane: 1 wait state (without
  it the read returns the register's previous contents; 2 are kept here);
* a transcendental (v_exp / v_log / v_rcp) result read by a non-
  transcendental VALU op: 1 wait state;
* an MFMA reading the previous MFMA's destination as its accumulator (same
  registers): no wait;
* an LDS read's destination: s_waitcnt lgkmcnt(n) with n = LDS ops issued
  after it (LDS ops complete in order; at most 15 are kept in flight).

Immediate offsets are range-checked: the assembler keeps only the low 12 bits
of a MUBUF `offset:` (and 16 of a DS one) without a diagnostic.

Each emitted instruction counts as one wait state, s_nop N as N + 1.  These
are the numbers the compiler itself inserts for gfx950 in the same
situations.
"""
from __future__ import annotations

import re

MFMA_TO_OTHER = 12
VALU_TO_MFMA = 2
VALU_TO_PERMLANE = 2
VALU_TO_READLANE = 2
TRANS_TO_VALU = 1
MAX_LGKM = 15


def expand(reg: str):
    """'v[4:7]' -> ['v4','v5','v6','v7'];  'a12' -> ['a12'];  's[2:3]' -> [...]"""
    m = re.fullmatch(r"([vas])\[(\d+):(\d+)\]", reg)
    if m:
        k, lo, hi = m.group(1), int(m.group(2)), int(m.group(3))
        return [f"{k}{i}" for i in range(lo, hi + 1)]
    m = re.fullmatch(r"([vas])(\d+)", reg)
    if m:
        return [reg]
    return []  # constants, vcc, exec, m0, literals


class Block:
    """A contiguous register range of one kind ('v', 'a' or 's')."""

    def __init__(self, kind: str, base: int, n: int, name: str = ""):
        self.kind, self.base, self.n, self.name = kind, base, n, name

    def r(self, i: int = 0, n: int = 1) -> str:
        assert 0 <= i and i + n <= self.n, (self.name, i, n, self.n)
        if n == 1:
            return f"{self.kind}{self.base + i}"
        return f"{self.kind}[{self.base + i}:{self.base + i + n - 1}]"

    def __str__(self):
        return self.r(0, self.n)


class Alloc:
    def __init__(self, kind: str, start: int, limit: int, align_multi: int = 1):
        self.kind, self.next, self.limit = kind, start, limit
        self.align_multi = align_multi
        self.blocks = {}

    def take(self, name: str, n: int, align: int = 1) -> Block:
        if n > 1 and self.align_multi > 1:
            align = max(align, self.align_multi)
        self.next = (self.next + align - 1) // align * align
        b = Block(self.kind, self.next, n, name)
        self.next += n
        assert self.next <= self.limit, f"out of {self.kind} registers at {name}: {self.next}"
        self.blocks[name] = b
        return b


class Emitter:
    serialize = False   # debugging aid: drain after every MFMA and LDS read

    def __init__(self):
        self.lines = []
        self.idx = 0                 # wait-state clock
        self.mfma_w = {}             # reg -> idx of the MFMA that wrote it
        self.valu_w = {}             # reg -> idx of the VALU write
        self.trans_w = {}            # reg -> idx of a transcendental write
        self.lds_pending = []        # list of sets of regs written by in-flight LDS reads
        self.n_mfma = self.n_valu = self.n_ds = 0

    # ---- bookkeeping ------------------------------------------------------
    def snapshot(self):
        return (self.idx, dict(self.mfma_w), dict(self.valu_w), dict(self.trans_w),
                [set(x) for x in self.lds_pending])

    def restore(self, snap):
        self.idx, self.mfma_w, self.valu_w, self.trans_w, pend = snap
        self.mfma_w, self.valu_w, self.trans_w = dict(self.mfma_w), dict(self.valu_w), dict(self.trans_w)
        self.lds_pending = [set(x) for x in pend]

    # ---- relative states, for control-flow joins ----------------------------
    def rel_state(self):
        """The hazard state as ages (wait states since each write) plus the
        in-flight LDS reads, independent of the absolute clock."""
        ages = tuple({r: self.idx - w for r, w in t.items()}
                     for t in (self.mfma_w, self.valu_w, self.trans_w))
        return ages, [set(x) for x in self.lds_pending]

    @staticmethod
    def merge_rel(a, b):
        """Conservative merge of two relative states: the most recent write of
        each register, and in-flight LDS reads aligned at the newest one."""
        ages = []
        for ta, tb in zip(a[0], b[0]):
            m = dict(ta)
            for r, v in tb.items():
                m[r] = min(m.get(r, v), v)
            ages.append(m)
        pa, pb = a[1], b[1]
        n = max(len(pa), len(pb))
        pend = []
        for i in range(n):
            sa = pa[len(pa) - n + i] if len(pa) - n + i >= 0 else set()
            sb = pb[len(pb) - n + i] if len(pb) - n + i >= 0 else set()
            pend.append(set(sa) | set(sb))
        return tuple(ages), pend

    def apply_rel(self, rel):
        ages, pend = rel
        self.mfma_w, self.valu_w, self.trans_w = (
            {r: self.idx - a for r, a in t.items()} for t in ages)
        self.lds_pending = [set(x) for x in pend][-MAX_LGKM:]

    def drain(self):
        """Make every earlier result safe to use (used at control-flow joins)."""
        if self.lds_pending:
            self._raw("s_waitcnt lgkmcnt(0)")
            self.lds_pending = []
        self._nop(MFMA_TO_OTHER)
        self.mfma_w.clear()
        self.valu_w.clear()
        self.trans_w.clear()

    def _raw(self, text: str, cost: int = 1):
        self.lines.append("\t" + text)
        self.idx += cost

    def label(self, name: str):
        self.lines.append(f"{name}:")

    def comment(self, text: str):
        self.lines.append(f"\t; {text}")

    def _nop(self, n: int):
        while n > 0:
            k = min(n, 16)
            self._raw(f"s_nop {k - 1}", cost=k)
            n -= k

    def _need(self, table, regs, states):
        """Pad so that at least `states` wait states separate the producer
        (at clock table[r]) from the instruction about to issue at self.idx;
        idx - table[r] - 1 instructions already lie between them."""
        worst = 0
        for r in regs:
            if r in table:
                worst = max(worst, table[r] + 1 + states - self.idx)
        if worst > 0:
            self._nop(worst)

    def _wait_lds(self, regs):
        regs = set(regs)
        hit = -1
        for i, ws in enumerate(self.lds_pending):
            if ws & regs:
                hit = i
        if hit >= 0:
            n = len(self.lds_pending)
            after = min(n - 1 - hit, MAX_LGKM)
            self._raw(f"s_waitcnt lgkmcnt({after})")
            self.lds_pending = self.lds_pending[n - after:] if after > 0 else []

    def _clear_writes(self, regs):
        for r in regs:
            self.mfma_w.pop(r, None)
            self.valu_w.pop(r, None)
            self.trans_w.pop(r, None)

    # ---- instruction kinds --------------------------------------------------
    def salu(self, text: str):
        self._raw(text)

    @staticmethod
    def _check_offset(text: str, limit: int):
        m = re.search(r"offset:(\d+)", text)
        assert m is None or int(m.group(1)) <= limit, f"immediate offset out of range: {text}"

    def valu(self, text: str, dst=(), src=(), trans=False):
        dregs = [x for d in dst for x in expand(d)]
        sregs = [x for s in src for x in expand(s)]
        self._wait_lds(sregs + dregs)
        self._need(self.mfma_w, sregs + dregs, MFMA_TO_OTHER)
        if not trans:
            self._need(self.trans_w, sregs, TRANS_TO_VALU)
        if text.startswith("v_permlane"):
            self._need(self.valu_w, sregs, VALU_TO_PERMLANE)
        if text.startswith(("v_readfirstlane", "v_readlane")):
            self._need(self.valu_w, sregs, VALU_TO_READLANE)
        self._raw(text)
        self._clear_writes(dregs)
        for r in dregs:
            self.valu_w[r] = self.idx - 1
            if trans:
                self.trans_w[r] = self.idx - 1
        self.n_valu += 1

    def mfma(self, op: str, d: str, a: str, b: str, c: str):
        """d = a * b + c.  c may be '0'."""
        dregs, aregs, bregs, cregs = expand(d), expand(a), expand(b), expand(c)
        srcs = aregs + bregs + cregs
        self._wait_lds(srcs)
        self._need(self.valu_w, srcs, VALU_TO_MFMA)
        # another MFMA's destination may only come back as this one's accumulator
        for r in aregs + bregs:
            assert r not in self.mfma_w, f"MFMA source {r} is a recent MFMA result"
        if cregs:
            assert cregs == dregs, "accumulator must be the destination"
        self._raw(f"{op} {d}, {a}, {b}, {c}")
        self._clear_writes(dregs)
        for r in dregs:
            self.mfma_w[r] = self.idx - 1
        self.n_mfma += 1
        if self.serialize:
            self._nop(64)

    def ds_read(self, text: str, dst: str, addr: str):
        dregs = expand(dst)
        self._wait_lds(dregs)           # WAW on a pending load's destination
        self._need(self.mfma_w, dregs + expand(addr), MFMA_TO_OTHER)
        self._check_offset(text, 65535)
        while len(self.lds_pending) >= MAX_LGKM:
            self._raw(f"s_waitcnt lgkmcnt({MAX_LGKM - 1})")
            self.lds_pending = self.lds_pending[1:]
        self._raw(text)
        self._clear_writes(dregs)
        self.lds_pending.append(set(dregs))
        self.n_ds += 1
        if self.serialize:
            self._raw("s_waitcnt lgkmcnt(0)")
            self.lds_pending = []

    def vmem(self, text: str, src=()):
        """buffer loads / stores; src = VGPR/AGPR operands read."""
        sregs = [x for s in src for x in expand(s)]
        self._wait_lds(sregs)
        self._need(self.mfma_w, sregs, MFMA_TO_OTHER)
        self._check_offset(text, 4095)
        self._raw(text)

    def vmem_load_to(self, text: str, dst: str, src=()):
        """buffer load whose destination registers are tracked only by vmcnt
        (the caller waits explicitly)."""
        dregs = expand(dst)
        sregs = [x for s in src for x in expand(s)]
        self._need(self.mfma_w, sregs + dregs, MFMA_TO_OTHER)
        self._check_offset(text, 4095)
        self._raw(text)
        self._clear_writes(dregs)

    def text(self) -> str:
        return "\n".join(self.lines) + "\n"


def interleave(em: Emitter, mfmas, others, lead: int = 0):
    """Emit two independent instruction streams, spreading `others` (callables
    emitting one instruction each) evenly between the `mfmas` (callables
    emitting one MFMA each).  `lead` MFMAs go first."""
    mf = list(mfmas)
    ot = list(others)
    i = 0
    for k in range(min(lead, len(mf))):
        mf[k]()
    mf = mf[lead:]
    n = len(mf)
    for k, f in enumerate(mf):
        f()
        remaining_m = n - k
        take = (len(ot) - i + remaining_m - 1) // remaining_m
        for _ in range(take):
            ot[i]()
            i += 1
    while i < len(ot):
        ot[i]()
        i += 1


class Op:
    """One schedulable instruction (or an indivisible group) with an issue
    cost in VALU-instruction units."""

    def __init__(self, fn, cost=1.0):
        self.fn, self.cost = fn, cost

    def __call__(self):
        self.fn()


def weave(em: Emitter, mfmas, others, tail: float = 0.0):
    """Spread `others` (Op objects, emitted in list order) over the gaps after
    each MFMA so that every gap carries about the same issue cost.  `tail`
    extra cost units are assumed to follow the last MFMA (work emitted after
    the call), so the last gaps are left lighter."""
    mf = list(mfmas)
    ot = list(others)
    total = sum(o.cost for o in ot) + tail
    n = len(mf)
    if n == 0:
        for o in ot:
            o()
        return
    per = total / n
    i, done = 0, 0.0
    for k, f in enumerate(mf):
        f()
        target = per * (k + 1)
        while i < len(ot) and done + ot[i].cost * 0.5 <= target:
            ot[i]()
            done += ot[i].cost
            i += 1
    while i < len(ot):
        ot[i]()
        i += 1
