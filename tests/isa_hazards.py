"""Static check of the library's gfx950 assembly for one hazard class.

A vector-ALU (or memory) instruction that reads or overwrites a register a
matrix (MFMA) op writes needs a number of wait states after the op (for the
8-pass 32x32x16 op, at least 11 issue slots; s_nop N counts N + 1) that the
hardware does not enforce.  The compiler inserts them, but its count follows
one control-flow path back to the op; where an exec-mask branch sits in
between, another path can reach the read sooner.  This checker walks every
path from every matrix op of every kernel and reports each instruction that
touches the op's destination registers with fewer wait states than required.
A chained matrix op that accumulates into the same registers (the hardware
interlocks those) ends a path.
"""
from __future__ import annotations

import re
from collections import defaultdict

NEED = 11


def regs_of(tok):
    tok = tok.strip().rstrip(',')
    m = re.match(r'^([av])\[(\d+):(\d+)\]$', tok)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {tok} if re.match(r'^[av]\d+$', tok) else set()


def functions(asm_text):
    """{kernel name: [("label", name) | ("ins", opcode, [operands])]}"""
    funcs, cur = {}, None
    for line in asm_text.splitlines():
        m = re.match(r'^(_Z\w+):', line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur is None:
            continue
        t = line.strip()
        if t == 's_endpgm':
            funcs[cur].append(("ins", "s_endpgm", []))
            cur = None
            continue
        m = re.match(r'^(\.LBB\w+):', line)
        if m:
            funcs[cur].append(("label", m.group(1), None))
            continue
        if not t or t.startswith((';', '.')):
            continue
        parts = t.split(None, 1)
        ops = [x.strip() for x in parts[1].split(',')] if len(parts) > 1 else []
        funcs[cur].append(("ins", parts[0], ops))
    return funcs


def _blocks(items):
    blocks, labels, cur = [], {}, []
    for kind, a, b in items:
        if kind == "label":
            if cur:
                blocks.append(cur)
            cur = []
            labels[a] = len(blocks)
            continue
        cur.append((a, b))
        if a.startswith('s_cbranch') or a in ('s_branch', 's_endpgm', 's_setpc_b64'):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    succ = defaultdict(list)
    for i, bl in enumerate(blocks):
        op, ops = bl[-1]
        if op.startswith('s_cbranch') or op == 's_branch':
            tgt = ops[0].split()[0]
            if tgt in labels:
                succ[i].append(labels[tgt])
            if op != 's_branch' and i + 1 < len(blocks):
                succ[i].append(i + 1)
        elif op != 's_endpgm' and i + 1 < len(blocks):
            succ[i].append(i + 1)
    return blocks, succ


def _touches(op, ops):
    """Registers an instruction reads, plus those a vector instruction writes."""
    stores = ('ds_write', 'global_store', 'buffer_store', 'flat_store', 'scratch_store')
    regs = set()
    for x in (ops if op.startswith(stores) else ops[1:]):
        regs |= regs_of(x)
    if op.startswith('v_') and ops and not op.startswith(('v_cmp', 'v_readfirstlane', 'v_readlane')):
        regs |= regs_of(ops[0])
    return regs


def hazards(items, need=NEED):
    """[(matrix op, its destination, offending instruction, wait states)] of one kernel."""
    blocks, succ = _blocks(items)
    found = []
    for bi, bl in enumerate(blocks):
        for ii, (op, ops) in enumerate(bl):
            if not op.startswith('v_mfma'):
                continue
            dst = regs_of(ops[0])
            best = {}
            stack = [(bi, ii + 1, 0)]
            while stack:
                b, k, w = stack.pop()
                if w >= need or best.get((b, k), need) <= w:
                    continue
                best[(b, k)] = w
                if k >= len(blocks[b]):
                    stack.extend((s, 0, w) for s in succ[b])
                    continue
                op2, ops2 = blocks[b][k]
                if op2.startswith('s_nop'):
                    stack.append((b, k + 1, w + 1 + int(ops2[0], 0)))
                    continue
                if op2.startswith('v_mfma'):
                    if regs_of(ops2[0]) & dst and len(ops2) >= 4 and regs_of(ops2[-1]) & dst:
                        continue                       # chained accumulation: interlocked
                    if set().union(*[regs_of(x) for x in ops2[1:3]]) & dst:
                        found.append((f"{op} {ops[0]}", f"{op2} {' '.join(ops2)}", w))
                        continue
                elif _touches(op2, ops2) & dst:
                    found.append((f"{op} {ops[0]}", f"{op2} {' '.join(ops2)}", w))
                    continue
                stack.append((b, k + 1, w + 1))
    return found
