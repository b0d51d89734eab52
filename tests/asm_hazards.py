"""Wait states between matrix-core results and their readers in compiled
gfx950 device code (the AMD assembly of this library's own build).

The matrix cores do not interlock every read of an MFMA result: the compiler
must place enough independent instructions (or s_nop) between an MFMA and a
VALU or memory instruction that reads its destination registers, on every
control-flow path.  A branch straight after score MFMAs was once compiled
with a single instruction on the path that skipped it, and the maxima read
stale registers.  `check_function` runs a forward dataflow over a kernel's
basic blocks: each MFMA sets its destination registers to `required` pending
wait states, every instruction retires one (s_nop N retires N + 1), joins
take the larger count, and a read of a register that still has pending wait
states is reported.
"""
from __future__ import annotations

import re

_REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")
_MEM = ("global_", "buffer_", "flat_", "ds_", "scratch_")


def _regs(text: str):
    out = []
    for m in _REG.finditer(text):
        if m.group(1):
            out += [f"{m.group(1)}{r}" for r in range(int(m.group(2)), int(m.group(3)) + 1)]
        else:
            out.append(f"{m.group(4)}{m.group(5)}")
    return out


def functions(asm: str, name_filter: str = "_kernel"):
    """(symbol, lines) of every function whose symbol contains name_filter."""
    lines = asm.split("\n")
    out = []
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\w*):", line)
        if m and name_filter in m.group(1):
            end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
            out.append((m.group(1), lines[i + 1:end]))
    return out


def _blocks(body):
    """Basic blocks: a label starts one, and so does the instruction after
    any branch (blocks that no branch targets carry no label in the asm)."""
    order, blocks, cur = ["<entry>"], {"<entry>": []}, "<entry>"
    for line in body:
        m = re.match(r"^(\.LBB\w+):", line)
        if m:
            cur = m.group(1)
            order.append(cur)
            blocks[cur] = []
            continue
        s = line.split(";")[0].strip()
        if not s or s.startswith("."):
            continue
        if blocks[cur] and blocks[cur][-1].startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            cur = f"<after {cur}>"
            order.append(cur)
            blocks[cur] = []
        blocks[cur].append(s)
    succ = {}
    for k, b in enumerate(order):
        last = blocks[b][-1] if blocks[b] else ""
        nxt = [order[k + 1]] if k + 1 < len(order) else []
        if last.startswith("s_branch"):
            succ[b] = [last.split()[1]]
        elif last.startswith("s_cbranch"):
            succ[b] = [last.split()[1]] + nxt
        elif last.startswith(("s_endpgm", "s_setpc")):
            succ[b] = []
        else:
            succ[b] = nxt
    return order, blocks, succ


def _reads(op: str, operands):
    """Vector registers an instruction reads (None: not a VALU/memory op)."""
    if op.startswith(_MEM):
        store = any(k in op for k in ("store", "write", "atomic"))
        src = operands if store else operands[1:]
    elif op.startswith("v_"):
        # accumulate forms and writelane also read their destination
        keep_dst = "mac" in op or op.startswith("v_writelane")
        src = operands if keep_dst else operands[1:]
    else:
        return None
    regs = []
    for o in src:
        regs += _regs(o)
    return regs


def check_function(body, required: int):
    """Reads of MFMA results with fewer than `required` wait states on some
    path: a list of (block, index, instruction, missing wait states)."""
    order, blocks, succ = _blocks(body)
    state_in = {b: {} for b in order}
    work = list(order)
    found = set()
    while work:
        b = work.pop(0)
        st = dict(state_in[b])
        for idx, ins in enumerate(blocks[b]):
            op = ins.split()[0]
            operands = ins[len(op):].split(",")
            retire = 1
            m = re.match(r"s_nop\s+(\d+)", ins)
            if m:
                retire = int(m.group(1)) + 1
            if "mfma" not in op:
                reads = _reads(op, operands)
                for r in reads or ():
                    if r in st:
                        found.add((b, idx, ins, st[r]))
            for r in list(st):
                st[r] -= retire
                if st[r] <= 0:
                    del st[r]
            if "mfma" in op:
                for r in _regs(operands[0]):
                    st[r] = required
        for s in succ[b]:
            if s not in state_in:
                continue
            merged, changed = dict(state_in[s]), False
            for r, v in st.items():
                if merged.get(r, 0) < v:
                    merged[r], changed = v, True
            if changed:
                state_in[s] = merged
                if s not in work:
                    work.append(s)
    return sorted(found)
