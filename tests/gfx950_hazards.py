"""Wait-state checker for gfx950 assembly listings (test infrastructure).

Hand-scheduled instruction streams must keep the software-managed hazard distances of the
CDNA3/CDNA4 matrix cores themselves; these are the ones the prefill stream relies on,
counted in wait states (one per issued instruction, N+1 for s_nop N) along every control
path:
  matrix-core result (vdst)       -> any non-matrix access of it          >= 12
  matrix-core result              -> srcA/B of a later matrix product     >= 12
  vector-ALU register write       -> read by a matrix product             >= 2
  exp2 / rcp / log / sqrt result  -> read by the next instruction         >= 1
  dot2 result                     -> read by another kind of instruction  >= 3
  permlane swap operands          -> any access after it                  >= 2
  M0 write                        -> direct-to-LDS load (reads M0)        >= 1
"""
import re

REG = re.compile(r'\b([vas])\[(\d+):(\d+)\]|\b([vas])(\d+)\b|\b(m0)\b')
TRANS = ('v_exp_f32', 'v_rcp_f32', 'v_log_f32', 'v_sqrt_f32', 'v_rsq_f32')


def regs(text):
    """Registers named in an operand string, as (file, index) pairs; m0 as ('m', 0)."""
    out = set()
    for m in REG.finditer(text):
        if m.group(1):
            out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        elif m.group(4):
            out.add((m.group(4), int(m.group(5))))
        else:
            out.add(('m', 0))
    return out


def parse(lines):
    """Instructions (op, operand list, text) and label -> index."""
    ins, labels = [], {}
    for ln in lines:
        s = ln.split(';')[0].strip()
        if not s or (s.startswith('.') and not s.endswith(':')):
            continue
        if s.endswith(':'):
            labels[s[:-1]] = len(ins)
            continue
        parts = s.split(None, 1)
        ops = [a.strip() for a in parts[1].split(',')] if len(parts) > 1 else []
        ins.append((parts[0], ops, s))
    return ins, labels


def _waits(op, ops):
    return int(ops[0], 0) + 1 if op == 's_nop' else 1


def _succ(i, ins, labels):
    op, ops, _ = ins[i]
    if op == 's_branch':
        out = [labels[ops[0]]]
    elif op.startswith('s_cbranch'):
        out = [labels[ops[0]], i + 1]
    elif op == 's_endpgm':
        out = []
    else:
        out = [i + 1]
    return [j for j in out if j < len(ins)]


def _walk(i, need, ins, labels, visit):
    """Call visit(j, w) for every instruction j reachable from i at fewer than `need`
    wait states (w = wait states before j)."""
    stack = [(j, 0) for j in _succ(i, ins, labels)]
    seen = set()
    while stack:
        j, w = stack.pop()
        if (j, w) in seen or w >= need:
            continue
        seen.add((j, w))
        visit(j, w)
        op2, ops2, _ = ins[j]
        stack += [(k, w + _waits(op2, ops2)) for k in _succ(j, ins, labels)]


def check(ins, labels):
    """List of (rule, i, j, wait_states, text_i, text_j) violations."""
    bad = []
    for i, (op, ops, s) in enumerate(ins):
        if op.startswith('v_mfma'):
            dst = regs(ops[0])

            def v_mfma(j, w, dst=dst, i=i, s=s):
                op2, ops2, s2 = ins[j]
                if op2.startswith('v_mfma'):
                    if dst & (regs(ops2[1]) | regs(ops2[2])):
                        bad.append(('mfma D -> mfma srcA/B', i, j, w, s, s2))
                    c2 = regs(ops2[3]) if len(ops2) > 3 else set()
                    if dst & c2 and c2 != dst:
                        bad.append(('mfma D -> partial srcC', i, j, w, s, s2))
                elif not op2.startswith('s_') and dst & regs(','.join(ops2)):
                    bad.append(('mfma D -> non-mfma access', i, j, w, s, s2))
            _walk(i, 12, ins, labels, v_mfma)
        elif op.startswith('v_') and ops and not op.startswith(('v_cmp', 'v_readfirstlane', 'v_readlane')):
            d = regs(ops[0])

            def v_valu(j, w, d=d, i=i, s=s):
                op2, ops2, s2 = ins[j]
                if op2.startswith('v_mfma') and d & regs(','.join(ops2[1:])):
                    bad.append(('valu write -> mfma read', i, j, w, s, s2))
            _walk(i, 2, ins, labels, v_valu)
        for prefix, need, name, exempt in ((TRANS, 1, 'trans -> read', None),
                                           (('v_dot2c', 'v_dot2_'), 3, 'dot -> read', 'v_dot2c'),
                                           (('v_permlane',), 2, 'permlane -> access', None)):
            if not op.startswith(prefix):
                continue
            d = regs(ops[0]) | (regs(ops[1]) if prefix[0] == 'v_permlane' else set())

            def v_read(j, w, d=d, i=i, s=s, name=name, exempt=exempt):
                op2, ops2, s2 = ins[j]
                if not op2.startswith(('v_', 'ds_', 'global_', 'buffer_')):
                    return
                srcs = ','.join(ops2[1:]) if op2.startswith('v_') and name != 'permlane -> access' else ','.join(ops2)
                if d & regs(srcs) and not (exempt and op2.startswith(exempt) and regs(ops2[0]) == d):
                    bad.append((name, i, j, w, s, s2))
            _walk(i, need, ins, labels, v_read)
        if op.startswith('s_') and ops and regs(ops[0]) == {('m', 0)}:
            def v_m0(j, w, i=i, s=s):
                op2, ops2, s2 = ins[j]
                lds_dma = op2.startswith('global_load_lds') or (op2.startswith('buffer_load') and
                                                                  s2.split()[-1] == 'lds')
                if lds_dma:
                    bad.append(('m0 write -> lds load', i, j, w, s, s2))
            _walk(i, 1, ins, labels, v_m0)
    return bad


def functions(listing_text):
    """name -> lines of each function in an assembly listing."""
    funcs, cur = {}, None
    for ln in listing_text.splitlines():
        m = re.match(r'^(_Z\S+):', ln)
        if m:
            cur = m.group(1)
            funcs[cur] = []
            continue
        if cur is not None:
            funcs[cur].append(ln)
            if 's_endpgm' in ln:
                cur = None
    return funcs
