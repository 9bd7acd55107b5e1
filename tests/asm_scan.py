"""Static check of the gfx950 assembly of the HIP kernels: an LDS read written
in inline assembly (`ds_read*` between the compiler's ;;#ASMSTART / ;;#ASMEND
markers) leaves its destination registers in flight until an
`s_waitcnt lgkmcnt` retires it, and the compiler, which does not know that,
may copy, spill or overwrite those registers in the meantime.  This scanner
follows every path through each kernel's control-flow graph and reports any
instruction that reads or writes a register of such a read before the wait.

Model: LDS reads retire in issue order, so lgkmcnt(N) retires all but the N
youngest reads on the path (kernels here issue no scalar loads between an LDS
read and its wait); the set of reads in flight at a block's entry is the
union over its predecessors.
"""
from __future__ import annotations

import re
from collections import defaultdict

_LABEL = re.compile(r"^(\.?[A-Za-z_$][\w.$]*):$")
_FUNC = re.compile(r"^(_Z\S*?):")


def _regs(tok: str) -> frozenset:
    tok = tok.strip().rstrip(",")
    m = re.fullmatch(r"([va])(\d+)", tok)
    if m:
        return frozenset({(m.group(1), int(m.group(2)))})
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return frozenset((m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1))
    return frozenset()


def _functions(lines):
    name, body = None, []
    for ln, raw in enumerate(lines, 1):
        st = raw.strip()
        m = _FUNC.match(st)
        if m:
            if name:
                yield name, body
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if st.startswith(".Lfunc_end"):
            yield name, body
            name, body = None, []
            continue
        body.append((ln, st))
    if name:
        yield name, body


def _blocks(body):
    blocks, name, insts, inasm = [], "<entry>", [], False
    for ln, st in body:
        if st.startswith(";;#ASMSTART"):
            inasm = True
            continue
        if st.startswith(";;#ASMEND"):
            inasm = False
            continue
        code = st.split(";")[0].strip()
        m = _LABEL.match(code)
        if m:
            blocks.append((name, insts))
            name, insts = m.group(1), []
            continue
        if not code or code.startswith("."):
            continue
        insts.append((ln, code, inasm))
        if code.startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            # a branch ends its block; the compiler prints the fall-through
            # block's name only as a comment
            blocks.append((name, insts))
            name, insts = f"<after line {ln}>", []
    blocks.append((name, insts))
    return blocks


def _successors(blocks):
    index = {n: i for i, (n, _) in enumerate(blocks)}
    succ = defaultdict(list)
    for i, (_, insts) in enumerate(blocks):
        last = insts[-1][1] if insts else ""
        op = last.split()[0] if last else ""
        if op == "s_branch":
            succ[i].append(index.get(last.split()[1]))
        elif op.startswith("s_cbranch"):
            succ[i].append(index.get(last.split()[1]))
            succ[i].append(i + 1 if i + 1 < len(blocks) else None)
        elif op not in ("s_endpgm", "s_setpc_b64"):
            succ[i].append(i + 1 if i + 1 < len(blocks) else None)
    return succ


def scan_function(body):
    """(read line, touching line, touching instruction) for every hazard."""
    blocks = _blocks(body)
    succ = _successors(blocks)
    entry_state = defaultdict(frozenset)
    found = set()
    work = list(range(len(blocks)))
    while work:
        i = work.pop(0)
        pend = sorted(entry_state[i], key=lambda x: x[1])
        for ln, code, inasm in blocks[i][1]:
            m = re.search(r"lgkmcnt\((\d+)\)", code)
            if code.startswith("s_waitcnt") and m:
                n = int(m.group(1))
                pend = pend[len(pend) - n:] if n else []
                continue
            parts = code.split(None, 1)
            ops = [o.split()[0] for o in re.split(r",\s*", parts[1]) if o.strip()] if len(parts) > 1 else []
            touched = frozenset().union(*[_regs(o) for o in ops]) if ops else frozenset()
            if parts[0].startswith("ds_read") and inasm and ops:
                srcs = frozenset().union(*[_regs(o) for o in ops[1:]]) if len(ops) > 1 else frozenset()
                for rs, src in pend:
                    if srcs & rs:
                        found.add((src, ln, code))
                pend.append((_regs(ops[0]), ln))
                continue
            for rs, src in pend:
                if touched & rs:
                    found.add((src, ln, code))
        out = frozenset(pend)
        for j in succ[i]:
            if j is None:
                continue
            merged = entry_state[j] | out
            if merged != entry_state[j]:
                entry_state[j] = merged
                if j not in work:
                    work.append(j)
    return sorted(found)


def scan_text(text: str):
    """{function: [(read line, touching line, instruction), ...]} for the
    functions of an assembly listing that have a hazard."""
    out = {}
    for name, body in _functions(text.splitlines()):
        hits = scan_function(body)
        if hits:
            out[name] = hits
    return out
