"""Static check of generated gfx950 assembly: every s_barrier must be reached with this
wave's LDS stores complete (an `s_waitcnt lgkmcnt(0)` after the last ds_write on every
path), or another wave can pass the barrier and read LDS the stores have not yet written.
The backend does not add that wait by itself on targets with back-off barriers; it comes
from the barrier's workgroup-release fence, which in one loop shape was placed so that
the back edge missed it. Works on the control-flow graph of each kernel."""

from __future__ import annotations

import re


def kernel_bodies(asm: str):
    """(name, instruction lines) of each kernel in an assembly listing."""
    out, cur = [], None
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\w+):", line)
        if m:
            cur = (m.group(1), [])
            out.append(cur)
        elif cur is not None:
            cur[1].append(line)
    return out


def _blocks(lines):
    blocks, labels, b = [], {}, None
    for ln in lines:
        s = ln.split(";")[0].strip()
        lm = re.match(r"^(\.LBB\w+):", ln.strip())
        if lm:
            b = {"label": lm.group(1), "ins": []}
            blocks.append(b)
            labels[lm.group(1)] = len(blocks) - 1
            continue
        if not s or s.startswith("."):
            continue
        if b is None:
            b = {"label": "entry", "ins": []}
            blocks.append(b)
        b["ins"].append(s)
        if s.startswith("s_endpgm"):
            break
    succ = []
    for i, bb in enumerate(blocks):
        sc, fall = set(), True
        for ins in bb["ins"]:
            op = ins.split()[0]
            if op.startswith("s_cbranch") or op == "s_branch":
                tgt = ins.split()[-1]
                if tgt in labels:
                    sc.add(labels[tgt])
                if op == "s_branch":
                    fall = False
            if op == "s_endpgm":
                fall = False
        if fall and i + 1 < len(blocks):
            sc.add(i + 1)
        succ.append(sc)
    return blocks, succ


def _step(pending: bool, ins: str) -> bool:
    op = ins.split()[0]
    if op.startswith("ds_") and ("write" in op or "store" in op):
        return True
    if op == "s_waitcnt" and re.search(r"lgkmcnt\(0\)", ins):
        return False
    return pending


def unsafe_barriers(lines) -> list[str]:
    """Labels of the blocks holding an s_barrier reachable with an LDS store not waited on."""
    blocks, succ = _blocks(lines)
    inn = [False] * len(blocks)
    changed = True
    while changed:
        changed = False
        for i, bb in enumerate(blocks):
            st = inn[i]
            for ins in bb["ins"]:
                st = _step(st, ins)
            for j in succ[i]:
                if st and not inn[j]:
                    inn[j] = changed = True
    bad = []
    for i, bb in enumerate(blocks):
        st = inn[i]
        for ins in bb["ins"]:
            if ins.split()[0] == "s_barrier" and st:
                bad.append(bb["label"])
            st = _step(st, ins)
    return sorted(set(bad))
