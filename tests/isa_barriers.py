"""Static check of compiled gfx950 assembly: can a wave reach `s_barrier` while
LDS reads it issued are still outstanding?

The kernels hand LDS buffers from one wave to another at barriers (a stage that
every wave has finished reading is refilled after the barrier). `s_barrier`
itself does not wait for a wave's outstanding LDS reads, and the compiler may
schedule the waits for them (with the instructions that use the data) below a
barrier. Such a read can then return data that another wave has already
overwritten. This module finds those barriers.

Method: the assembly of each kernel is split into basic blocks (labels,
branches, `s_endpgm`); the number of LDS reads that may be outstanding is
propagated along the control-flow graph (maximum over predecessors, iterated
to a fixed point). `ds_read*` adds one; `s_waitcnt ... lgkmcnt(n)` caps the
count at n (LDS operations complete in order). A barrier reached with a
non-zero count is reported.
"""
from __future__ import annotations

import re
from dataclasses import dataclass

_LABEL = re.compile(r"^(\.LBB\d+_\d+):")
_BRANCH = re.compile(r"^s_(branch|cbranch_\w+)\s+(\.LBB\d+_\d+)")
_LGKM = re.compile(r"lgkmcnt\((\d+)\)")
_CAP = 64


@dataclass
class Finding:
    kernel: str
    block: str
    outstanding: int


def _kernels(text: str):
    """Yield (name, instruction lines) per kernel function in the assembly."""
    name, body = None, []
    for raw in text.splitlines():
        line = raw.split(";")[0].rstrip()
        m = re.match(r"^([A-Za-z_][\w.$]*):\s*$", line)
        if m and not line.startswith("."):
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if re.match(r"^\.Lfunc_end\d+:", line.strip()):
            yield name, body
            name, body = None, []
            continue
        body.append(line.strip())


def _blocks(lines):
    blocks, cur, label = [], [], "entry"
    for t in lines:
        if not t:
            continue
        m = _LABEL.match(t)
        if m:
            if label is not None:
                blocks.append((label, cur))
            label, cur = m.group(1), []
            continue
        if t.startswith("."):
            continue                       # directives
        if label is None:                  # code after an unconditional jump
            label, cur = f"_anon{len(blocks)}", []
        cur.append(t)
        if t.startswith("s_endpgm") or t.startswith("s_branch") or t.startswith("s_setpc"):
            blocks.append((label, cur))
            label, cur = None, []
        elif t.startswith("s_cbranch"):
            blocks.append((label, cur))
            label, cur = f"_ft{len(blocks)}", []
    if label is not None:
        blocks.append((label, cur))
    return blocks


def _transfer(count: int, ins) -> int:
    for t in ins:
        if t.startswith("ds_read"):
            count = min(count + 1, _CAP)
        elif t.startswith("s_waitcnt"):
            m = _LGKM.search(t)
            if m:
                count = min(count, int(m.group(1)))
    return count


def barrier_hazards(asm_text: str) -> list[Finding]:
    """Barriers that some path reaches with LDS reads of the same wave in flight."""
    found = []
    for kname, lines in _kernels(asm_text):
        blocks = _blocks(lines)
        index = {lab: i for i, (lab, _) in enumerate(blocks)}
        succ = []
        for i, (_, ins) in enumerate(blocks):
            last = ins[-1] if ins else ""
            nxt = []
            m = _BRANCH.match(last)
            if m and m.group(2) in index:
                nxt.append(index[m.group(2)])
            ends = last.startswith("s_branch") or last.startswith("s_endpgm") or last.startswith("s_setpc")
            if not ends and i + 1 < len(blocks):
                nxt.append(i + 1)
            succ.append(nxt)
        entry = [0] * len(blocks)
        changed = True
        while changed:
            changed = False
            for i, (_, ins) in enumerate(blocks):
                out = _transfer(entry[i], ins)
                for j in succ[i]:
                    if out > entry[j]:
                        entry[j] = out
                        changed = True
        for i, (lab, ins) in enumerate(blocks):
            count = entry[i]
            for t in ins:
                if t.startswith("s_barrier") and count:
                    found.append(Finding(kname, lab, count))
                count = _transfer(count, [t])
    return found


def kernel_count(asm_text: str) -> int:
    return sum(1 for _ in _kernels(asm_text))
