"""Scan of gfx950 assembly for the MFMA hazards the compiler cannot see
through inline assembly (used by test_asm_hazards.py).

Two rules, with wait states counted as one per instruction in between and
N+1 for ``s_nop N``:
  * a vector (VALU) instruction that writes a register read by a following
    MFMA as any operand needs 2 wait states before that MFMA;
  * a vector instruction that reads or writes a register written by a
    preceding MFMA needs the wait states the kernels place by hand (16).
"""

import re

READ_AFTER_VALU = 2
AFTER_MFMA = 16


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _instructions(lines):
    out = []
    for line in lines:
        t = line.split(";")[0].strip()
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        op, _, rest = t.partition(" ")
        out.append((op, [o.strip().split()[0] for o in rest.split(",") if o.strip()] if rest else []))
    return out


def _wait_states(op, ops):
    if op == "s_nop":
        return int(ops[0], 0) + 1 if ops else 1
    return 1


def findings(lines):
    """Hazards in one function's assembly lines, as readable strings."""
    ins = _instructions(lines)
    found = []
    for i, (op, ops) in enumerate(ins):
        if not op.startswith("v_mfma") or len(ops) < 4:
            continue
        dst = _regs(ops[0])
        srcs = set().union(*(_regs(o) for o in ops[1:4]))
        ws = 0
        for j in range(i - 1, -1, -1):
            pop, pops = ins[j]
            if pop.startswith("v_") and not pop.startswith("v_mfma") and pops and _regs(pops[0]) & srcs:
                found.append("%s %s -> %s after %d wait states" % (pop, pops[0], op, ws))
                break
            ws += _wait_states(pop, pops)
            if ws >= READ_AFTER_VALU or pop.startswith("s_cbranch") or pop.startswith("s_branch"):
                break
        ws = 0
        for j in range(i + 1, len(ins)):
            pop, pops = ins[j]
            if pop.startswith("v_") and not pop.startswith("v_mfma"):
                if set().union(*(_regs(o) for o in pops)) & dst:
                    found.append("%s %s -> %s after %d wait states" % (op, ops[0], pop, ws))
                    break
            if pop.startswith("s_cbranch") or pop.startswith("s_branch") or pop.startswith("s_endpgm"):
                break
            ws += _wait_states(pop, pops)
            if ws >= AFTER_MFMA:
                break
    return found


def scan(text):
    """{function name: [findings]} for every function in an assembly file."""
    lines = text.split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_Z\S+:", l)]
    result = {}
    for k, s in enumerate(starts):
        e = starts[k + 1] if k + 1 < len(starts) else len(lines)
        result[lines[s].split(":")[0]] = findings(lines[s + 1:e])
    return result
