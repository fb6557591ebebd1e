"""Scan of gfx950 assembly for reads of MFMA results too close to the MFMA.

For every MFMA, finds the nearest instruction on any control path (through branches) that reads
its destination registers other than as the accumulator input of another MFMA.  The distance
counts issued instructions, s_nop N as N + 1.  A read one instruction after the MFMA, on the path
where a data-dependent branch skips an MFMA block, has given silently stale values."""
import re
import sys


def min_read_distance(asm: str, pattern: str, limit: int = 12):
    """{kernel symbol: (distance, mfma line, reader line)} for the kernels whose symbol contains pattern."""
    out = {}
    s = asm
    pat = pattern
    LIMIT = limit
    def regs(tok):
        m = re.match(r'([va])\[(\d+):(\d+)\]', tok)
        if m: return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
        m = re.match(r'([va])(\d+)$', tok)
        if m: return {(m.group(1), int(m.group(2)))}
        return set()
    for m in re.finditer(r'^(_Z\w+):\s*;', s, re.M):
        name = m.group(1)
        if pat not in name: continue
        start = m.end(); end = s.index('.Lfunc_end', start)
        lines = [l.split(';')[0].strip() for l in s[start:end].splitlines()]
        ins, labels = [], {}
        for l in lines:
            if not l or l.startswith('.') and not l.endswith(':'): continue
            if l.endswith(':'): labels[l[:-1]] = len(ins); continue
            ins.append(l)
        def ops(l):
            parts = l.split(None, 1)
            return parts[0], ([t.strip() for t in parts[1].split(',')] if len(parts) > 1 else [])
        worst = (99, None)
        for i, l in enumerate(ins):
            op, a = ops(l)
            if not op.startswith('v_mfma'): continue
            dst = regs(a[0])
            # BFS along paths
            stack = [(i + 1, 0)]; seen = set()
            while stack:
                j, d = stack.pop()
                if d >= LIMIT or j >= len(ins) or (j, d) in seen: continue
                seen.add((j, d))
                op2, a2 = ops(ins[j])
                if op2.startswith('v_mfma'):
                    srcs = a2[1:3]
                    if any(regs(t) & dst for t in srcs):
                        worst = min(worst, (d, (i, l, j, ins[j])))
                    if regs(a2[0]) & dst and not (regs(a2[3]) & dst if len(a2) > 3 else False):
                        pass
                    stack.append((j + 1, d + 1)); continue
                reads = a2[1:] if not op2.startswith(('s_', 'ds_write', 'global_store', 'buffer_store')) else a2
                if op2.startswith(('ds_write', 'global_store', 'buffer_store')): reads = a2
                if any(regs(t) & dst for t in reads):
                    worst = min(worst, (d, (i, l, j, ins[j])))
                    continue
                step = int(a2[0]) + 1 if op2 == 's_nop' else 1
                if op2.startswith('s_endpgm'): continue
                if op2.startswith('s_branch'):
                    stack.append((labels[a2[0]], d + step)); continue
                if op2.startswith('s_cbranch'):
                    stack.append((labels[a2[0]], d + step))
                stack.append((j + 1, d + step))
        out[name] = (worst[0], worst[1][1] if worst[1] else None, worst[1][3] if worst[1] else None)
    return out


if __name__ == "__main__":
    for k, v in min_read_distance(open(sys.argv[1]).read(), sys.argv[2]).items():
        print(k[:70], v[0])
