"""Dataflow check of gfx9 assembly for LDS reads used before they land.

An LDS read (ds_read*) returns its data some cycles after it issues; the
destination registers may be read or written only after an
`s_waitcnt lgkmcnt(N)` has covered the load.  The compiler inserts those
waits for the loads it emits itself, but not for loads written as inline asm,
and it does not know that their destinations are still in flight: it may
copy or reuse them early.  This module finds every such use.

The hardware rule it applies: LDS operations complete in issue order, so a
read with at least N LDS operations issued after it is complete once
`s_waitcnt lgkmcnt(N)` passes (scalar memory loads also count on lgkmcnt but
may complete in any order; they are therefore never credited with pushing an
LDS read out).  The state at each point is, per register, the least number
of LDS operations issued after the newest pending read into it; states of
several predecessors of a block merge by taking the least number (the most
conservative), and the analysis iterates over the control-flow graph to a
fixed point.

An LDS read may overwrite the destination of an older pending read (they
land in order); any other instruction that names a pending destination,
as source or destination, is a hazard.
"""
import re

REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")
LGKM = re.compile(r"lgkmcnt\((\d+)\)")
BRANCH = re.compile(r"^s_(?:c)?branch\w*\s+(\.LBB\w+)")
CAP = 16   # lgkmcnt is a 4-bit field on gfx9: a read 16 LDS operations old is always covered


def regs(text):
    """Vector (v) and accumulation (a) registers named in an operand string."""
    out = set()
    for kind, lo, hi, one in REG.findall(text):
        if one:
            out.add(f"{kind}{one}")
        else:
            out.update(f"{kind}{i}" for i in range(int(lo), int(hi) + 1))
    return out


def split(ins):
    """(mnemonic, operand text) of one instruction line."""
    ins = ins.split(";")[0].strip()
    parts = ins.split(None, 1)
    return (parts[0], parts[1] if len(parts) > 1 else "") if parts else ("", "")


def lgkm_wait(mn, ops):
    """The lgkmcnt an s_waitcnt waits for, or None if it does not wait on it."""
    if mn != "s_waitcnt":
        return None
    m = LGKM.search(ops)
    if m:
        return int(m.group(1))
    ops = ops.strip()
    if re.fullmatch(r"(0x[0-9a-fA-F]+|\d+)", ops):   # raw immediate: lgkmcnt in bits 11:8
        return (int(ops, 0) >> 8) & 15
    return None


def is_lds_read(mn):
    return mn.startswith("ds_read") or mn in ("ds_bpermute_b32", "ds_permute_b32", "ds_swizzle_b32")


def transfer(ins_list, state, hazards=None, where=None):
    """Apply a block's instructions to a state (register -> LDS operations
    since its pending read); record hazards if a list is given."""
    st = dict(state)
    for idx, ins in enumerate(ins_list):
        mn, ops = split(ins)
        if not mn:
            continue
        n = lgkm_wait(mn, ops)
        if n is not None:
            st = {r: d for r, d in st.items() if d < n}
            continue
        if is_lds_read(mn):
            dest_text, _, src_text = ops.partition(",")
            dest = regs(dest_text)
            bad = regs(src_text) & st.keys()
        else:
            dest = set()
            bad = regs(ops) & st.keys()
        if bad and hazards is not None:
            hazards.append((where, idx, ins.strip(), sorted(bad)))
        if mn.startswith("ds_"):
            st = {r: min(d + 1, CAP) for r, d in st.items()}
            for r in dest:
                st[r] = 0
    return st


def cfg(blocks):
    """Successor indices of each block (layout order; a block falls through
    to the next unless it ends in an unconditional branch or returns)."""
    index = {label.split(":")[0]: i for i, (label, _) in enumerate(blocks)}
    succ = []
    for i, (_, ins) in enumerate(blocks):
        s = []
        last = ""
        for x in ins:
            mn, _ = split(x)
            if not mn:
                continue
            last = mn
            m = BRANCH.match(x.strip())
            if m and m.group(1) in index:
                s.append(index[m.group(1)])
        if last not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    return succ


def merge(a, b):
    out = dict(a)
    for r, d in b.items():
        out[r] = min(out.get(r, CAP), d)
    return out


def hazards(blocks):
    """Every instruction of a function (blocks: [(label, [instruction])] in
    layout order, the entry first) that uses the destination of an LDS read
    not yet covered by a wait: [(block label, index, instruction, registers)]."""
    succ = cfg(blocks)
    ins_state = [None] * len(blocks)
    ins_state[0] = {}
    work = [0]
    while work:
        i = work.pop()
        out = transfer(blocks[i][1], ins_state[i])
        for j in succ[i]:
            new = out if ins_state[j] is None else merge(ins_state[j], out)
            if new != ins_state[j]:
                ins_state[j] = new
                work.append(j)
    found = []
    for i, (label, ins) in enumerate(blocks):
        if ins_state[i] is not None:
            transfer(ins, ins_state[i], found, label.split(":")[0])
    return found


def functions(asm, name_pattern):
    """name -> [(block label, [instruction])] for each function whose symbol
    matches name_pattern (a regex)."""
    lines = asm.split("\n")
    out = {}
    i = 0
    while i < len(lines):
        m = re.match(rf"^({name_pattern}):", lines[i])
        if not m:
            i += 1
            continue
        name = m.group(1)
        blocks, cur = [], ("entry", [])
        i += 1
        unnamed = 0
        while i < len(lines) and not lines[i].startswith(".Lfunc_end"):
            ln = lines[i]
            if re.match(r"^\.LBB\w+:", ln):
                blocks.append(cur)
                cur = (ln, [])
            elif ln.startswith("\t") and not ln.strip().startswith((";", ".")):
                cur[1].append(ln.strip())
                if split(ln)[0].startswith(("s_branch", "s_cbranch")):
                    # A basic block ends at a branch; the assembler prints
                    # no label for a block that is only fallen into.
                    blocks.append(cur)
                    unnamed += 1
                    cur = (f".unnamed{unnamed}", [])
            i += 1
        blocks.append(cur)
        out[name] = blocks
    return out
