"""Dataflow check of inline-asm vector loads in gfx950 assembly (run by the
build on every compile of the GEMM kernels, and by the tests).

The GEMM kernels issue every load through compiler builtins, so the build
requires that none of them contains an inline-asm vector load.  The hazard
this guards against: a load written as inline asm (`global_load_dwordx4`
waited for by an explicit `s_waitcnt vmcnt(n)`) is invisible to the
compiler's own wait insertion.  The compiler takes an asm
output as written when the asm statement ends, but the hardware writes the
register only when the load returns.  So until a wait has drained the load,
the compiler must not read, copy, spill or reuse that register.  If it does,
the copy holds stale data, and the late write lands in a register that may by
then hold something else (an address, say).

This module finds every register that may still be the target of an asm load
in flight, at every instruction of a function, by forward dataflow over the
function's control-flow graph:
  * an asm load adds its destination registers to the in-flight set;
  * `s_waitcnt vmcnt(0)` (or a bare `s_waitcnt 0`) empties it;
  * partial waits leave it as it is (conservative: which loads a partial
    wait retires is checked separately, against the issue order);
  * the in-flight sets of a block's predecessors are merged by union.
An instruction that names an in-flight register is a violation, except for
the two intended uses: the data operand of `ds_write_b128` (the loader's
store, placed after its partial wait) and the destination of another asm
load.  Spill instructions (`scratch_*`) in the region are violations too.
"""
import re

_BRANCH = re.compile(r"^s_(c?branch|endpgm|setpc)")
_LABEL = re.compile(r"^(\.LBB\d+_\d+):")


def vgprs(text):
    """The VGPR numbers an operand string names (v7, v[4:7])."""
    out = set()
    for a, b in re.findall(r"\bv\[(\d+):(\d+)\]", text):
        out.update(range(int(a), int(b) + 1))
    rest = re.sub(r"\bv\[\d+:\d+\]", "", text)
    out.update(int(x) for x in re.findall(r"\bv(\d+)\b", rest))
    return out


def functions(asm_text):
    """{symbol: [lines]} for every function in an assembly listing."""
    funcs, cur = {}, None
    for line in asm_text.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur and line.startswith(".Lfunc_end"):
            cur = None
            continue
        if cur:
            funcs[cur].append(line)
    return funcs


def _instructions(lines):
    ins, in_asm = [], False
    for line in lines:
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not t or t.startswith(";") or (t.startswith(".") and not _LABEL.match(t)):
            continue
        ins.append((t.split(";")[0].strip(), in_asm))
    return ins


def _blocks(ins):
    blocks, order, lab, n = {"entry": []}, ["entry"], "entry", 0
    for t, a in ins:
        m = _LABEL.match(t)
        if m:
            lab = m.group(1)
            blocks[lab] = []
            order.append(lab)
            continue
        blocks[lab].append((t, a))
        if _BRANCH.match(t):  # a branch ends its block; what follows starts a new one
            n += 1
            lab = "after%d" % n
            blocks[lab] = []
            order.append(lab)
    succ = {}
    for i, b in enumerate(order):
        s, falls = [], True
        for t, _ in blocks[b]:
            m = re.match(r"^s_branch\s+(\S+)", t)
            if m:
                s.append(m.group(1))
                falls = False
            m = re.match(r"^s_cbranch_\w+\s+(\S+)", t)
            if m:
                s.append(m.group(1))
            if t.startswith("s_endpgm") or t.startswith("s_setpc"):
                falls = False
        if falls and i + 1 < len(order):
            s.append(order[i + 1])
        succ[b] = s
    return blocks, order, succ


def _drains(t):
    if not t.startswith("s_waitcnt"):
        return False
    if re.search(r"vmcnt\(0\)", t):
        return True
    return re.match(r"^s_waitcnt\s+0$", t) is not None


def analyse(lines):
    """(number of asm vector loads, [violating instructions]) for one function."""
    blocks, order, succ = _blocks(_instructions(lines))
    live_in = {b: set() for b in order}
    bad = {}
    changed = True
    while changed:
        changed = False
        for b in order:
            st = set(live_in[b])
            for t, in_asm in blocks[b]:
                op = t.split(None, 1)[0]
                if in_asm and op.startswith("global_load"):
                    ops = t.split(None, 1)[1].split(",")
                    if vgprs(",".join(ops[1:])) & st:  # address operand still in flight
                        bad[t] = b
                    st |= vgprs(ops[0])
                    continue
                if _drains(t):
                    st = set()
                    continue
                if op == "ds_write_b128":
                    addr = t.split(None, 1)[1].split(",")[0]
                    if vgprs(addr) & st:
                        bad[t] = b
                    continue
                if (vgprs(t) & st) or op.startswith("scratch_"):
                    bad[t] = b
            for s in succ[b]:
                if not st <= live_in[s]:
                    live_in[s] |= st
                    changed = True
    n = sum(1 for b in order for t, a in blocks[b] if a and t.startswith("global_load"))
    return n, sorted(bad)


def check_loader_asm(asm_text, expected_functions=0):
    """Raise RuntimeError unless every function with inline-asm loads leaves
    their registers alone until a wait drains them, and exactly
    `expected_functions` functions issue such loads (none in the library's
    kernels).  Returns the number of functions checked."""
    checked, problems = 0, []
    for name, lines in functions(asm_text).items():
        n, bad = analyse(lines)
        if n == 0:
            continue
        checked += 1
        if bad:
            problems.append("%s: %d instructions touch in-flight load registers, e.g. %s" % (name, len(bad), bad[:3]))
    if problems:
        raise RuntimeError("loader register hazard in the GEMM kernels:\n" + "\n".join(problems))
    if checked != expected_functions:
        raise RuntimeError("expected %d GEMM instantiations with inline-asm loads, found %d" %
                           (expected_functions, checked))
    return checked
