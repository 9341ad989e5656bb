"""Static check of the built library's gfx950 code for LDS results touched
before they have landed.

An LDS read (ds_read*, and the other LDS operations that return data) writes
its destination registers when it completes, some cycles after it issues; the
program must wait for it (s_waitcnt lgkmcnt(n): at most n LDS operations still
outstanding, and LDS operations complete in issue order) before any other
instruction reads or writes those registers.  Reads issued from inline
assembly are invisible to the compiler's own wait insertion: if it copies their
results before the wait the source code places after them, the copy takes the
registers' old contents.

The check walks each kernel's control flow (fall-through and branch targets)
forward, with the list of outstanding LDS operations and their destination
registers as the state (merged over incoming paths), and reports every
instruction that touches a register an outstanding LDS operation will still
write.  Scalar memory loads also count in lgkmcnt but may complete out of order,
so they are left out: a wait then retires at least the LDS operations this
assumes.
"""
import re

from mfma_hazards import _operands, _regs

MAX_OUTSTANDING = 64


def _has_result(op):
    return op.startswith("ds_") and any(w in op for w in ("read", "load", "permute", "swizzle", "_rtn"))


def _successors(ins):
    index = {a: i for i, (a, _) in enumerate(ins)}
    succ = [[] for _ in ins]
    for i, (a, t) in enumerate(ins):
        op = t.split()[0]
        m = re.match(r"s_c?branch\S*\s+(-?\d+)", t)
        if m:
            off = int(m.group(1))
            if off > 32767:
                off -= 65536
            tgt = a + 4 + 4 * off
            if tgt in index:
                succ[i].append(index[tgt])
        if op not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(ins):
            succ[i].append(i + 1)
    return succ


def _merge(a, b):
    """Outstanding lists aligned at the newest operation; registers united."""
    n = max(len(a), len(b))
    a = (frozenset(),) * (n - len(a)) + a
    b = (frozenset(),) * (n - len(b)) + b
    return tuple(x | y for x, y in zip(a, b))


def _step(t, state, report):
    op = t.split()[0]
    if op == "s_waitcnt":
        m = re.search(r"lgkmcnt\((\d+)\)", t)
        if m:
            n = int(m.group(1))
            state = state[len(state) - n:] if 0 < n < len(state) else (state if n else ())
        return state
    if op.startswith("s_"):
        return state
    ops = _operands(t)
    touched = set()
    for o in (ops[1:] if _has_result(op) else ops):
        touched |= _regs(o)
    for pending in state:
        if pending & touched:
            report(pending & touched)
    if _has_result(op):
        state = (state + (frozenset(_regs(ops[0])),))[-MAX_OUTSTANDING:]
    elif op.startswith("ds_"):
        state = (state + (frozenset(),))[-MAX_OUTSTANDING:]
    return state


def early_lds_uses(ins):
    """[instruction text] of one kernel that touch an outstanding LDS result."""
    succ = _successors(ins)
    entry = {0: ()} if ins else {}
    work = list(entry)
    found = set()
    while work:
        i = work.pop()
        state = entry[i]
        hits = []
        state = _step(ins[i][1], state, hits.append)
        if hits:
            found.add(i)
        for j in succ[i]:
            old = entry.get(j)
            new = state if old is None else _merge(old, state)
            if new != old:
                entry[j] = new
                work.append(j)
    return [ins[i][1] for i in sorted(found)]
