"""Scan gfx950 assembly for reads of MFMA results issued too soon after the MFMA.

A VALU instruction (v_accvgpr_read included) that reads registers an XDL MFMA wrote
must come enough wait states later; the hardware does not interlock it.  The
v_mfma_f32_32x32x16_bf16 used here needs 11 (8 passes + 3).  The scan walks every
control-flow path from each MFMA -- fallthrough and branch targets, forward and
backward -- for up to that many wait states and reports any path that reaches a
read of the MFMA's destination first.  It found a real miscompile: a short taken
branch between an MFMA chain and its accumulator reads left 5 wait states.
"""
import re


def scan(asm_text, min_wait=11):
    """List of human-readable hazard reports (empty when the code is safe)."""
    lines = [l.rstrip() for l in asm_text.splitlines()]
    return _scan(lines, min_wait)


def _scan(lines, MIN):
    insts = []   # (text, label or None)
    labels = {}
    fn = None
    for l in lines:
        t = l.strip()
        if not t or t.startswith(';') or t.startswith('.') and not re.match(r'^\.LBB', t):
            continue
        m = re.match(r'^(\.LBB[\w_]+):', t)
        if m:
            labels[m.group(1)] = len(insts); continue
        if re.match(r'^[_A-Za-z][\w.$]*:', t):   # function label
            insts.append(("<fn " + t + ">", None)); continue
        insts.append((t.split(';')[0].strip(), None))
    def regs(spec):
        out = set()
        m = re.match(r'([av])\[(\d+):(\d+)\]', spec)
        if m:
            return {m.group(1) + str(i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        m = re.match(r'([av])(\d+)$', spec)
        if m: return {spec}
        return out
    def ws(t):
        m = re.match(r's_nop (\d+)', t)
        return int(m.group(1)) + 1 if m else 1
    def reads(t):
        parts = t.replace(',', ' ').split()
        if len(parts) < 2: return set()
        r = set()
        for p in parts[2:]:
            r |= regs(p)
        return r
    bad = []
    for i, (t, _) in enumerate(insts):
        if not t.startswith('v_mfma'): continue
        dst = regs(t.replace(',', ' ').split()[1])
        # paths: list of (position, waitstates so far)
        frontier = [(i + 1, 0)]
        seen = set()
        while frontier:
            pos, w = frontier.pop()
            while pos < len(insts) and w < MIN:
                tt = insts[pos][0]
                if tt.startswith('<fn'): break
                if tt.startswith('v_mfma'):
                    # a dependent MFMA (srcC) is interlocked by hardware; stop this path at a rewrite
                    if dst & regs(tt.replace(',', ' ').split()[1]): break
                elif dst & reads(tt):
                    bad.append(f"{w} wait states from [{t}] to [{tt}]"); break
                m = re.match(r's_cbranch_\w+ (\.LBB[\w_]+)|s_branch (\.LBB[\w_]+)', tt)
                w += ws(tt)
                if m:
                    tgt = labels.get(m.group(1) or m.group(2))
                    if tgt is not None and (tgt, w) not in seen:
                        seen.add((tgt, w)); frontier.append((tgt, w))
                    if tt.startswith('s_branch'): break
                pos += 1
    return bad
