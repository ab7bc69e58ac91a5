"""Static checks of the built gfx950 ISA of kernels that issue MFMAs and LDS reads as inline
assembly, which the compiler does not track.

Two properties are checked on every control-flow path of each kernel:

1. MFMA register dependencies (`mfma_hazards`).  The compiler resolves them for builtin MFMAs
   but cannot see an inline-assembly MFMA as one:
   - no VALU instruction writes a register an MFMA reads (A, B or C) within `before` wait
     states before the MFMA;
   - no non-MFMA instruction reads or writes an MFMA's result within `after` wait states after
     it, and no MFMA reads it as A or B in that window (back-to-back accumulation into the same
     registers as C is resolved by the hardware);
   - no instruction writes the C registers of an MFMA whose C differs from its result within
     `after` wait states after it.
   Wait states: one per instruction, N + 1 for `s_nop N`.  The windows are margins over what a
   32x32x16 product needs.

2. Untracked LDS reads (`early_lds_uses`): the registers an LDS read writes are not read or
   written by any instruction before an `s_waitcnt lgkmcnt(N)` with N at most the number of LDS
   operations issued after that read (LDS reads complete in order, so such a wait covers it).
   Compiler-tracked reads satisfy this by construction.

`check_sources` compiles the device code of the given sources to assembly and runs both checks;
the build calls it for the kernels whose MFMAs are inline assembly.
"""
import os
import re
import subprocess

MFMA_BEFORE = 4     # wait states between a VALU write of an operand and the MFMA
MFMA_AFTER = 20     # wait states between an MFMA and another access to its result or C


def _regs(tok):
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"^([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def kernel_names(asm):
    return re.findall(r"^(_Z\S+):", asm, re.M)


def parse(asm, name):
    """Instructions (op, operands, text) of one kernel and its label positions."""
    i = asm.index(name + ":")
    j = asm.index(".Lfunc_end", i)
    insts, labels = [], {}
    for line in asm[i:j].split("\n")[1:]:
        t = line.split(";")[0].strip()
        m = re.match(r"^(\.LBB\S+):", line)
        if m:
            labels[m.group(1)] = len(insts)
            continue
        if not t or t.startswith(".") or t.endswith(":"):
            continue
        op = t.split()[0]
        rest = t[len(op):]
        ops = [o.strip() for o in rest.split(",")] if rest.strip() else []
        insts.append((op, ops, t))
    return insts, labels


def _succs(insts, labels, k):
    op, ops, _ = insts[k]
    if op == "s_branch":
        return [labels[ops[0]]]
    if op.startswith("s_cbranch"):
        return [k + 1, labels[ops[0]]]
    if op == "s_endpgm":
        return []
    return [k + 1]


def _preds(insts, labels):
    p = {k: [] for k in range(len(insts) + 1)}
    for k in range(len(insts)):
        for n in _succs(insts, labels, k):
            p.setdefault(n, []).append(k)
    return p


def _wait_states(inst):
    op, ops, _ = inst
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def _is_mfma(op):
    return op.startswith("v_mfma")


def _valu_dst(inst):
    op, ops, _ = inst
    if not op.startswith("v_") or _is_mfma(op) or not ops:
        return set()
    return _regs(ops[0])


def _reads(inst):
    op, ops, _ = inst
    writes_first = not (op.startswith(("ds_write", "buffer_store", "global_store", "s_")))
    r = set()
    for o in ops[1 if writes_first else 0:]:
        for t in o.split():
            r |= _regs(t)
    return r


def _load_dst(inst):
    op, ops, _ = inst
    if ops and op.startswith(("ds_read", "buffer_load", "global_load", "scratch_load")):
        return _regs(ops[0])
    return set()


def mfma_hazards(asm, name, before=MFMA_BEFORE, after=MFMA_AFTER):
    insts, labels = parse(asm, name)
    preds = _preds(insts, labels)
    found = {}
    for k, (op, ops, txt) in enumerate(insts):
        if not _is_mfma(op):
            continue
        dst, a, b = _regs(ops[0]), _regs(ops[1]), _regs(ops[2])
        c = _regs(ops[3]) if len(ops) > 3 else set()
        # VALU writes of an operand shortly before the MFMA
        stack, seen = [(k, 0)], set()
        while stack:
            pos, acc = stack.pop()
            for p in preds.get(pos, []):
                if (p, acc) in seen:
                    continue
                seen.add((p, acc))
                if _valu_dst(insts[p]) & (a | b | c):
                    found[(k, p)] = ("operand written before", txt, insts[p][2])
                    continue
                if acc + _wait_states(insts[p]) < before:
                    stack.append((p, acc + _wait_states(insts[p])))
        # accesses to the result, and writes of a separate C, shortly after
        stack, seen = [(k, 0)], set()
        while stack:
            pos, acc = stack.pop()
            for n in _succs(insts, labels, pos):
                if n >= len(insts) or (n, acc) in seen:
                    continue
                seen.add((n, acc))
                op2, ops2, t2 = insts[n]
                hit = None
                if _is_mfma(op2):
                    a2, b2 = _regs(ops2[1]), _regs(ops2[2])
                    c2 = _regs(ops2[3]) if len(ops2) > 3 else set()
                    d2 = _regs(ops2[0])
                    chain = c2 == dst and d2 == dst
                    if (a2 | b2) & dst or (c2 & dst and not chain) or (d2 & dst and not chain):
                        hit = "result used by a product"
                else:
                    if (_reads(insts[n]) | _valu_dst(insts[n]) | _load_dst(insts[n])) & dst:
                        hit = "result accessed"
                    elif c != dst and (_valu_dst(insts[n]) | _load_dst(insts[n])) & c:
                        hit = "accumulator input overwritten"
                if hit:
                    found[(k, n)] = (hit, txt, t2)
                    continue
                if acc + _wait_states(insts[n]) < after:
                    stack.append((n, acc + _wait_states(insts[n])))
    return [(k, n) + v for (k, n), v in sorted(found.items())]


def early_lds_uses(asm, name):
    insts, labels = parse(asm, name)
    found = []
    for k, (op, ops, txt) in enumerate(insts):
        if not op.startswith("ds_read"):
            continue
        dst = _regs(ops[0])
        stack, seen = [(k, 0)], set()
        while stack:
            pos, younger = stack.pop()
            for n in _succs(insts, labels, pos):
                if n >= len(insts) or (n, younger) in seen:
                    continue
                seen.add((n, younger))
                op2, ops2, t2 = insts[n]
                if op2 == "s_waitcnt":
                    m = re.search(r"lgkmcnt\((\d+)\)", t2)
                    if m and int(m.group(1)) <= younger:
                        continue
                touched = _reads(insts[n]) | _valu_dst(insts[n]) | _load_dst(insts[n])
                if _is_mfma(op2):
                    touched |= _regs(ops2[0])
                if touched & dst:
                    found.append((k, n, txt, t2))
                    continue
                issued = op2.startswith("ds_") or op2.startswith(("s_load", "s_buffer_load"))
                stack.append((n, min(younger + (1 if issued else 0), 64)))
    return found


def device_asm(src, flags, hipcc, out):
    cmd = [hipcc, *flags, "--cuda-device-only", "-S", "-x", "hip", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr}")
    return out


def check_asm(asm, mfma=True):
    """Findings per kernel of one assembly file: {name: [finding, ...]} (empty when clean)."""
    bad = {}
    for name in kernel_names(asm):
        f = (mfma_hazards(asm, name) if mfma else []) + early_lds_uses(asm, name)
        if f:
            bad[name] = f
    return bad


def check_sources(srcs, flags, hipcc, out_dir, mfma=True):
    """Compiles each source's device code to assembly in out_dir and checks it; raises on any
    finding."""
    report = []
    for src in srcs:
        out = os.path.join(out_dir, os.path.basename(src) + ".s")
        asm = open(device_asm(src, flags, hipcc, out)).read()
        for name, f in check_asm(asm, mfma).items():
            report.append(f"{os.path.basename(src)} {name}: {len(f)} finding(s), first: {f[0]}")
    if report:
        raise RuntimeError("ISA check failed:\n" + "\n".join(report))
