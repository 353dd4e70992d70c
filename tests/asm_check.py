"""Static check of gfx950 kernel assembly: no instruction touches the
destination registers of an LDS read before an ``s_waitcnt lgkmcnt`` has
retired that read.

The fat FFN kernels issue their operand LDS reads as inline assembly, so
that the compiler does not make them wait for the direct-to-LDS loads of
later pipeline stages.  The compiler then takes the read's result as ready
at once: under register pressure it may copy or spill the destination
registers (a ``v_mov``, ``v_accvgpr_write`` or ``scratch_store``) before the
wait that the source places after the read, and the copy holds stale data.
This checker walks the control-flow graph of each kernel and reports every
read or overwrite of a register whose LDS read may still be in flight on
some path.

LDS returns in issue order, so ``lgkmcnt(N)`` retires all but the newest N
LGKM operations -- unless a scalar memory load is among them (those return
out of order); then only ``lgkmcnt(0)`` retires anything here.
"""
import re

_REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")
_LGKM = re.compile(r"lgkmcnt\((\d+)\)")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.update(f"{m.group(1)}{r}" for r in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add(m.group(4) + m.group(5))
    return out


def _split_operands(rest):
    rest = rest.split(";")[0].strip()
    if not rest:
        return []
    return [o.strip() for o in re.split(r",(?![^\[]*\])", rest)]


def kernel_bodies(asm_text):
    """{symbol: [lines]} for every kernel function in an assembly file."""
    out, cur, name = {}, None, None
    for line in asm_text.split("\n"):
        m = re.match(r"^(_Z\S+):\s*(;.*)?$", line)
        if m:
            name, cur = m.group(1), []
            out[name] = cur
            continue
        if cur is not None:
            cur.append(line)
            if line.strip().startswith(".Lfunc_end"):
                cur = None
    return out


def _parse(lines):
    """Basic blocks: list of dicts with instructions and successor labels."""
    blocks, labels = [], {}

    def new(name):
        blocks.append({"name": name, "ins": [], "succ": [], "fall": True})
        return blocks[-1]

    cur = new("<entry>")
    for ln, raw in enumerate(lines, 1):
        s = raw.split(";")[0].strip() if not raw.strip().startswith(";;#ASM") else ""
        if not s:
            continue
        if s.endswith(":"):
            cur = new(s[:-1])
            labels[s[:-1]] = len(blocks) - 1
            continue
        if s.startswith("."):
            continue
        op = s.split()[0]
        ops = _split_operands(s[len(op):])
        cur["ins"].append((ln, op, ops, raw.strip()))
        if op == "s_branch":
            cur["succ"].append(ops[0])
            cur["fall"] = False
            cur = new(f"<after {ln}>")
        elif op.startswith("s_cbranch"):
            cur["succ"].append(ops[0])
            cur = new(f"<after {ln}>")
        elif op in ("s_endpgm", "s_setpc_b64"):
            cur["fall"] = False
            cur = new(f"<after {ln}>")
    succ = []
    for i, b in enumerate(blocks):
        ss = [labels[x] for x in b["succ"] if x in labels]
        if b["fall"] and i + 1 < len(blocks):
            ss.append(i + 1)
        succ.append(ss)
    return blocks, succ


def _step(state, ins, report):
    """Apply one instruction to the in-flight state (older, recent): `older`
    holds operations whose relative order is unknown (they reached a join
    from different paths), `recent` the ones issued since, oldest first.
    Each operation is (registers, line, is_scalar_load)."""
    older, recent = state
    ln, op, ops, raw = ins
    if op == "s_waitcnt":
        m = _LGKM.search(raw)
        if m:
            n = int(m.group(1))
            if n == 0:
                return (frozenset(), ())
            smem = any(x[2] for x in older) or any(x[2] for x in recent)
            if not smem and len(recent) >= n:
                return (frozenset(), recent[len(recent) - n:])
        return state
    if op.startswith("s_load") or op.startswith("s_buffer_load"):
        return (older, recent + ((frozenset(), ln, True),))
    is_store = "store" in op or op.startswith("ds_write") or op.startswith("buffer_store")
    dst = set() if (is_store or op.startswith("s_") or not ops) else _regs(ops[0])
    srcs = ops if is_store else ops[1:]
    used = set().union(*[_regs(o) for o in srcs]) if srcs else set()
    if report is not None and not op.startswith("s_"):
        for regs, rl, _ in list(older) + list(recent):
            hit = (used | dst) & regs
            if hit:
                report.append((ln, raw, rl, sorted(hit)[:4]))
    if op.startswith("ds_read") or op.startswith("ds_load"):
        return (older, recent + ((frozenset(_regs(ops[0])), ln, False),))
    if op.startswith("ds_") or op.startswith("s_sendmsg"):
        return (older, recent + ((frozenset(), ln, False),))
    return state


def _merge(a, b):
    if a == b:
        return a
    return (a[0] | b[0] | frozenset(a[1]) | frozenset(b[1]), ())


def stale_lds_uses(lines):
    """[(line, instruction, line of the LDS read, registers)] for one kernel."""
    blocks, succ = _parse(lines)
    empty = (frozenset(), ())
    entry = [None] * len(blocks)
    entry[0] = empty
    exit_ = [None] * len(blocks)
    work = [0]
    while work:
        i = work.pop()
        st = entry[i]
        for ins in blocks[i]["ins"]:
            st = _step(st, ins, None)
        if exit_[i] == st:
            continue
        exit_[i] = st
        for j in succ[i]:
            merged = st if entry[j] is None else _merge(entry[j], st)
            if merged != entry[j]:
                entry[j] = merged
                work.append(j)
    report = []
    for i, b in enumerate(blocks):
        if entry[i] is None:
            continue
        st = entry[i]
        for ins in b["ins"]:
            st = _step(st, ins, report)
    return report
