"""Static check of the wait states around inline-assembly MFMAs in generated gfx950 assembly.

The prefill tile kernel writes its MFMAs as inline assembly (accumulators updated in place in AGPRs),
so the compiler inserts no wait states for them; the kernel places them itself.  Two rules are checked
on every path of the control-flow graph (loop back-edges included):

  R1  an MFMA reads no VGPR (A or B operand) written by a vector-ALU instruction fewer than 2 wait
      states earlier;
  R2  no instruction other than an MFMA reads or writes an MFMA's accumulator AGPRs within 18 wait
      states after it.

A wait state is one instruction; `s_nop N` counts N + 1.
"""
from __future__ import annotations

import re

_REG = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")
_BRANCH = re.compile(r"^(s_branch|s_cbranch_\w+)\s+(\.?\w+)")


def _regs(text: str, kind: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            if m.group(1) == kind:
                out.add(int(m.group(2)))
        elif m.group(3) == kind:
            out.update(range(int(m.group(4)), int(m.group(5)) + 1))
    return out


class Inst:
    __slots__ = ("op", "args", "text")

    def __init__(self, text: str):
        self.text = text
        parts = text.split(None, 1)
        self.op = parts[0]
        self.args = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []

    @property
    def waits(self) -> int:
        if self.op == "s_nop":
            return int(self.args[0], 0) + 1
        return 1

    @property
    def is_mfma(self) -> bool:
        return self.op.startswith("v_mfma")

    def valu_vgpr_writes(self) -> set:
        if not self.op.startswith("v_") or self.is_mfma or not self.args:
            return set()
        return _regs(self.args[0], "v")


def functions(asm: str):
    """{kernel name: [Inst or label str]} of an assembly file."""
    funcs, cur = {}, None
    for raw in asm.splitlines():
        line = raw.split(";", 1)[0].strip()
        if not line or line.startswith(".") and not line.endswith(":"):
            continue
        if line.endswith(":"):
            name = line[:-1]
            if not name.startswith(".") and not name.startswith("$"):
                cur = funcs.setdefault(name, [])
                continue
            if cur is not None:
                cur.append(name)
            continue
        if cur is not None:
            cur.append(Inst(line))
    return funcs


def _cfg(items):
    """Instructions, and the successor and predecessor lists of each instruction index."""
    insts, label_at, pending = [], {}, []
    for it in items:
        if isinstance(it, str):
            pending.append(it)
        else:
            for lb in pending:
                label_at[lb] = len(insts)
            pending = []
            insts.append(it)
    n = len(insts)
    succ = [[] for _ in range(n)]
    for i, ins in enumerate(insts):
        m = _BRANCH.match(ins.text)
        if m and m.group(2) in label_at:
            succ[i].append(label_at[m.group(2)])
        if ins.op not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < n:
            succ[i].append(i + 1)
    pred = [[] for _ in range(n)]
    for i, ss in enumerate(succ):
        for j in ss:
            pred[j].append(i)
    return insts, succ, pred


def check(items, r1_waits: int = 2, r2_waits: int = 18):
    """List of (rule, index, instruction text, offending text, wait states between) violations."""
    insts, succ, pred = _cfg(items)
    bad = []
    for i, ins in enumerate(insts):
        if not ins.is_mfma or len(ins.args) < 3:
            continue
        srcs = _regs(ins.args[1], "v") | _regs(ins.args[2], "v")
        # R1: walk back until r1_waits wait states have passed on every path
        stack, seen = [(p, 0) for p in pred[i]], set()
        while stack:
            j, w = stack.pop()
            if (j, w) in seen or w >= r1_waits:
                continue
            seen.add((j, w))
            if insts[j].valu_vgpr_writes() & srcs:
                bad.append(("R1", i, ins.text, insts[j].text, w))
                continue
            stack.extend((p, w + insts[j].waits) for p in pred[j])
        # R2: walk forward until r2_waits wait states have passed on every path
        acc = _regs(ins.args[0], "a")
        stack, seen = [(s, 0) for s in succ[i]], set()
        while stack:
            j, w = stack.pop()
            if (j, w) in seen or w >= r2_waits:
                continue
            seen.add((j, w))
            other = insts[j]
            if not other.is_mfma and _regs(" ".join(other.args), "a") & acc:
                bad.append(("R2", i, ins.text, other.text, w))
                continue
            stack.extend((s, w + other.waits) for s in succ[j])
    return bad
