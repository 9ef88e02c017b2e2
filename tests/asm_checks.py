"""Checks on the gfx950 assembly of the decode kernel (test infrastructure).

The decode kernel issues its MFMAs, query loads and LDS copies as inline asm,
which the compiler neither schedules around nor protects with wait states or
wait counts.  These checks read the compiled assembly and verify what the
kernel's comments promise:
  * no VALU instruction writes an MFMA operand (or result register) less than
    two wait states before the MFMA;
  * no VALU instruction reads or writes a VGPR an MFMA writes less than 19
    wait states after the MFMA (the longest MFMA-result latency);
  * the registers of the asynchronous query and page-id loads are not touched
    between the load and the first explicit vmcnt wait after it;
  * every vmcnt wait in the decode kernel is one the source writes explicitly
    (the compiler adds none: an extra one would serialize the copy pipeline);
  * no VALU instruction overwrites the data registers of a preceding store of
    more than 8 bytes in the next wait state (gfx9-family store data hazard;
    the asm stores carry their own s_nop);
  * no VALU write of an SGPR is followed within 5 wait states by a vector
    memory instruction reading that SGPR (the asm copies take SGPR bases);
  * nothing but the next MFMA of the same accumulation chain reads or writes
    an MFMA's destination registers within 19 wait states (the matrix unit
    writes its result long after issue; a register the compiler reused right
    after an asm MFMA would race with that write).
The last two are for kernels whose MFMAs are inline asm: for MFMAs the
compiler emits itself it inserts the exact, shape-specific wait states.
"""
from __future__ import annotations

import re

DECODE_PREFIX = "_ZN3mla12_GLOBAL__N_113decode_kernel"


def _regs(tok: str) -> set:
    tok = tok.strip().rstrip(",")
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _split(line: str):
    t = line.split(";")[0].strip()
    parts = t.split(None, 1)
    if not parts:
        return "", []
    if len(parts) == 1:
        return parts[0], []
    return parts[0], [o.strip() for o in parts[1].split(",")]


def kernel_bodies(asm: str, prefix: str = DECODE_PREFIX, whole: bool = False) -> list:
    """Instruction lines of every function whose symbol starts with prefix (up
    to its first s_endpgm, or with ``whole`` to the end of the function)."""
    lines = asm.split("\n")
    out = []
    for i, l in enumerate(lines):
        if l.startswith(prefix) and l.split(";")[0].rstrip().endswith(":"):
            body = []
            for t in lines[i + 1 :]:
                if (".Lfunc_end" in t) if whole else ("s_endpgm" in t):
                    break
                t = t.strip()
                if not t or t.startswith(";") or t.startswith(".") or t.endswith(":"):
                    continue
                body.append(t)
            out.append(body)
    return out


def mfma_hazards(body: list) -> list:
    """(valu, mfma) pairs closer than two wait states (linear scan)."""
    bad = []
    for i, t in enumerate(body):
        op, ops = _split(t)
        if not op.startswith("v_mfma"):
            continue
        touched = set()
        for o in ops:
            touched |= _regs(o)
        need, j = 2, i - 1
        while need > 0 and j >= 0:
            pop, pops = _split(body[j])
            if pop == "s_nop":
                need -= int(pops[0], 0) + 1
                j -= 1
                continue
            if pop.startswith("v_") and not pop.startswith(("v_mfma", "v_readlane", "v_readfirstlane", "v_cmp")):
                written = _regs(pops[0]) if pops else set()
                if pop.startswith("v_permlane"):
                    for o in pops[:2]:
                        written |= _regs(o)
                if written & touched:
                    bad.append((body[j], t))
                    break
            need -= 1
            j -= 1
    return bad


def mfma_result_hazards(body: list, need: int = 19) -> list:
    """(mfma, valu) pairs where VALU touches an MFMA's VGPR result too early."""
    bad = []
    for i, t in enumerate(body):
        op, ops = _split(t)
        if not op.startswith("v_mfma") or not ops or not ops[0].startswith("v"):
            continue
        dst = _regs(ops[0])
        left, j = need, i + 1
        while left > 0 and j < len(body):
            uop, uops = _split(body[j])
            if uop == "s_nop":
                left -= int(uops[0], 0) + 1
                j += 1
                continue
            if uop.startswith("v_") and not uop.startswith("v_mfma"):
                if any(_regs(o) & dst for o in uops):
                    bad.append((t, body[j]))
                    break
            left -= 1
            j += 1
    return bad


def async_load_violations(body: list) -> list:
    """Instructions that touch an asm query load's registers before the next vmcnt wait."""
    bad = []
    for i, t in enumerate(body):
        op, ops = _split(t)
        if op not in ("global_load_dwordx4", "global_load_dword") or len(ops) < 2 or ops[-1] != "off":
            continue
        dst = _regs(ops[0])
        for u in body[i + 1 :]:
            if re.match(r"s_waitcnt\b.*vmcnt", u):
                break
            uop, uops = _split(u)
            if uop.startswith("global_load"):
                continue
            if any(_regs(o) & dst for o in uops):
                bad.append((t, u))
                break
    return bad


def store_data_hazards(body: list, need: int = 1) -> list:
    """(store, valu) pairs where VALU writes a 12/16-byte store's data registers too soon."""
    bad = []
    for i, t in enumerate(body):
        op, ops = _split(t)
        if not re.match(r"(global|buffer|flat)_store_dwordx[34]$", op) or len(ops) < 2:
            continue
        data = _regs(ops[1])
        left, j = need, i + 1
        while left > 0 and j < len(body):
            uop, uops = _split(body[j])
            if uop == "s_nop":
                left -= int(uops[0], 0) + 1
                j += 1
                continue
            if uop.startswith("v_") and uops:
                written = _regs(uops[0])
                if uop.startswith("v_permlane"):
                    for o in uops[:2]:
                        written |= _regs(o)
                if written & data:
                    bad.append((t, body[j]))
                    break
            left -= 1
            j += 1
    return bad


def vmcnt_waits(body: list) -> list:
    return [t for t in body if re.match(r"s_waitcnt\b", t) and "vmcnt" in t]


def pending_load_violations(body: list) -> list:
    """Instructions that touch the destination registers of a vector-memory load
    still outstanding under an in-order vmcnt model: loads and stores count up,
    `s_waitcnt vmcnt(N)` retires the oldest until N remain.  Catches the use of
    an inline-asm load (which the compiler does not wait for) before an
    explicit wait covers it.  Linear in layout order."""
    pending = []  # destination registers of outstanding operations, oldest first
    bad = []
    for t in body:
        m = re.match(r"s_waitcnt\b.*vmcnt\((\d+)\)", t)
        if m:
            del pending[: max(0, len(pending) - int(m.group(1)))]
            continue
        op, ops = _split(t)
        live = set().union(*pending) if pending else set()
        if op.startswith(("global_", "buffer_")):
            is_load = "load" in op and "_lds_" not in op
            srcs = ops[1:] if is_load else ops
            if any(_regs(o) & live for o in srcs) or (is_load and ops and _regs(ops[0]) & live):
                bad.append(t)
            pending.append(_regs(ops[0]) if is_load and ops else set())
            continue
        if any(_regs(o) & live for o in ops):
            bad.append(t)
    return bad


def _function_lines(asm: str, prefix: str) -> list:
    """Raw lines (comments kept) of every function whose symbol starts with prefix."""
    lines = asm.split("\n")
    out = []
    for i, l in enumerate(lines):
        if l.startswith(prefix) and l.split(";")[0].rstrip().endswith(":"):
            body = []
            for t in lines[i + 1 :]:
                if ".Lfunc_end" in t:
                    break
                body.append(t)
            out.append(body)
    return out


def compiler_agpr_uses(asm: str, prefix: str) -> list:
    """Instructions outside inline-asm blocks (;;#ASMSTART .. ;;#ASMEND) that
    name an accumulation register.  The decode kernels keep their output
    accumulators in AGPRs that only their inline asm touches; an instruction
    the compiler generated itself that reads or writes an a-register would
    mean the allocator placed something there (clobber lists do not reserve
    registers between asm statements)."""
    bad = []
    for body in _function_lines(asm, prefix):
        inside = False
        for l in body:
            s = l.strip()
            if s.startswith(";;#ASMSTART"):
                inside = True
                continue
            if s.startswith(";;#ASMEND"):
                inside = False
                continue
            t = s.split(";")[0].strip()
            if inside or not t or t.startswith(".") or t.endswith(":"):
                continue
            op, ops = _split(t)
            if op and any(re.match(r"a(\d+|\[\d+:\d+\])$", o) for o in ops):
                bad.append(t)
    return bad


def kernel_resources(asm: str) -> dict:
    """Per kernel symbol: spilled VGPRs/SGPRs and private (scratch) bytes, from
    the code object metadata."""
    res = {}
    cur = None
    for l in asm.split("\n"):
        s = l.strip()
        m = re.match(r"\.name:\s+(\S+)", s)
        if m:
            cur = m.group(1)
            res.setdefault(cur, {})
            continue
        if cur is None:
            continue
        for key in ("vgpr_spill_count", "sgpr_spill_count", "private_segment_fixed_size"):
            m = re.match(r"\." + key + r":\s+(\d+)", s)
            if m:
                res[cur][key] = int(m.group(1))
    return res


def _sgprs(tok: str) -> set:
    tok = tok.strip().rstrip(",")
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    if m:
        return {int(m.group(1))}
    if tok == "vcc":
        return {106, 107}
    if tok in ("vcc_lo", "vcc_hi"):
        return {106 if tok == "vcc_lo" else 107}
    return set()


def _wait_states(op: str, ops: list) -> int:
    if op == "s_nop":
        return int(ops[0], 0) + 1 if ops else 1
    return 1


def sgpr_vmem_hazards(body: list, need: int = 5) -> list:
    """A VALU write of an SGPR (v_readfirstlane, v_readlane, v_cmp to an SGPR
    pair, a carry out) followed by a vector-memory instruction that reads that
    SGPR as an address or offset needs `need` wait states in between (gfx9
    family).  The compiler inserts them between its own instructions but does
    not look inside inline asm, and the LDS copies and stores are inline asm
    taking SGPR bases.  Returns (index, vmem line, writer line) per violation."""
    bad = []
    last_write = {}  # sgpr -> (wait-state position after the writer, line)
    pos = 0
    for i, line in enumerate(body):
        op, ops = _split(line)
        if op.startswith(("global_", "buffer_", "flat_", "scratch_")):
            for o in (w for o in ops for w in o.split()):
                for s in _sgprs(o):
                    if s in last_write and pos - last_write[s][0] < need:
                        bad.append((i, line, last_write[s][1]))
        if op.startswith("v_") and not op.startswith(("v_mfma", "v_accvgpr")) and ops:
            dests = [ops[0]]
            if "_co_" in op or "div_scale" in op:
                dests.append(ops[1] if len(ops) > 1 else "")
            for d in dests:
                for s in _sgprs(d):
                    last_write[s] = (pos + 1, line)
        elif op.startswith("s_") and ops and not op.startswith(("s_waitcnt", "s_nop", "s_cbranch", "s_branch", "s_barrier")):
            # an SALU write clears the VALU-write record of that SGPR
            for s in _sgprs(ops[0]):
                last_write.pop(s, None)
        pos += _wait_states(op, ops)
    return bad


def _all_regs(tok: str) -> set:
    out = set()
    for w in tok.split():
        out |= _regs(w)
    return out


def mfma_dst_races(body: list, need: int = 19) -> list:
    """Instructions that read or write an MFMA's destination registers (VGPR or
    AGPR) within `need` wait states of the MFMA, other than a following MFMA
    that takes exactly that destination as its accumulator (srcC) and writes
    it again (an accumulation chain, which the hardware interlocks).  The
    matrix unit writes its result many cycles after issue; the compiler does
    not know an inline-asm MFMA's latency, so a register it considers free
    right after the asm, or a read that it schedules next to it, would race
    with that late write.  Returns (mfma line, racing line) pairs."""
    bad = []
    for i, t in enumerate(body):
        op, ops = _split(t)
        if not op.startswith("v_mfma") or len(ops) < 4:
            continue
        dst = _all_regs(ops[0])
        left, j = need, i + 1
        while left > 0 and j < len(body):
            uop, uops = _split(body[j])
            if uop == "s_nop":
                left -= int(uops[0], 0) + 1
                j += 1
                continue
            regs = [_all_regs(o) for o in uops]
            if uop.startswith("v_mfma") and len(uops) >= 4:
                chain = regs[3] == dst and regs[0] == dst
                if not chain and any(r & dst for r in regs):
                    bad.append((t, body[j]))
                    break
            elif any(r & dst for r in regs):
                bad.append((t, body[j]))
                break
            left -= 1
            j += 1
    return bad
