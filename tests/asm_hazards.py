"""Scan of gfx950 assembly for hazards the compiler cannot see.

The exact-path kernel issues its matrix products as inline asm, so the
compiler neither knows their latency nor inserts the wait states the CDNA
hazard rules require around them.  This scan checks the compiled assembly for
the two cases that bit us:

* a read or write of an inline-asm MFMA's result registers (VALU, memory,
  register copies) too soon after the MFMA issued: fewer than ``RESULT_WAITS``
  wait states, counting an ``s_nop k`` as k + 1, an intervening MFMA as 32
  (the matrix pipe takes a 32x32x16 product's passes before it accepts the
  next) and any other instruction as 1;
* a VALU write (including ``v_accvgpr_*`` copies) of an inline-asm MFMA's
  operand registers fewer than ``OPERAND_WAITS`` wait states before it.

Pending hazards follow branches to their targets (a second pass covers
backward branches).  Compiler-scheduled MFMAs (outside ``;;#ASMSTART`` /
``;;#ASMEND``) are not tracked: the compiler handles those itself.
"""

import re

RESULT_WAITS = 12
OPERAND_WAITS = 3
_REG = re.compile(r"\b([va])\[(\d+):(\d+)\]|\b([va])(\d+)\b")


def _regs(text):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
        else:
            out.add((m.group(4), int(m.group(5))))
    return out


def _age(items, n, limit):
    return [[d, w + n, l0] for d, w, l0 in items if w + n < limit]


def _merge(dst, items):
    for x in items:
        if x not in dst:
            dst.append(list(x))


def _scan(lines, at_label, report):
    pending, recent, in_asm = [], [], False
    for i, raw in enumerate(lines):
        stripped = raw.strip()
        if stripped.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if stripped.startswith(";;#ASMEND"):
            in_asm = False
            continue
        s = raw.split(";")[0].strip()
        if s.endswith(":"):  # a label (local ones start with '.')
            pending += [list(x) for x in at_label.get(("P", s[:-1]), [])]
            recent += [list(x) for x in at_label.get(("R", s[:-1]), [])]
            continue
        if not s or s.startswith("."):
            continue
        op = s.split()[0]
        rest = s[len(op):]
        if op.startswith(("s_branch", "s_cbranch")):
            tgt = rest.split(",")[0].strip()
            _merge(at_label.setdefault(("P", tgt), []), pending)
            _merge(at_label.setdefault(("R", tgt), []), recent)
            if op == "s_branch":
                pending, recent = [], []
            continue
        if op == "s_endpgm":
            pending, recent = [], []
            continue
        ops = [o.strip() for o in rest.split(",")]
        if op.startswith("v_mfma"):
            srcs_ab = _regs(",".join(ops[1:3]))
            for d, w, l0 in pending:
                if srcs_ab & d:
                    report(i, f"MFMA operand reads the result of the MFMA at line {l0 + 1} "
                              f"after {w} wait states")
            if in_asm:
                srcs = _regs(",".join(ops[1:]))
                for d, w, l0 in recent:
                    if srcs & d:
                        report(i, f"inline-asm MFMA reads {sorted(srcs & d)[:2]} written by "
                                  f"the VALU at line {l0 + 1} after {w} wait states")
            pending = _age(pending, 32, RESULT_WAITS)
            recent = _age(recent, 32, OPERAND_WAITS)
            if in_asm:
                pending.append([_regs(ops[0]), 0, i])
            continue
        if op == "s_nop":
            k = int(rest.strip(), 0) + 1
            pending = _age(pending, k, RESULT_WAITS)
            recent = _age(recent, k, OPERAND_WAITS)
            continue
        if op.startswith(("ds_write", "global_store", "scratch_store", "buffer_store", "s_")):
            used = _regs(rest)
        else:
            used = _regs(",".join(ops[1:])) | (_regs(ops[0]) if ops and ops[0] else set())
        for d, w, l0 in pending:
            if used & d:
                report(i, f"'{s}' touches {sorted(used & d)[:2]} of the MFMA at line "
                          f"{l0 + 1} after {w} wait states")
        pending = _age(pending, 1, RESULT_WAITS)
        recent = _age(recent, 1, OPERAND_WAITS)
        if op.startswith("v_") and ops and ops[0]:
            recent.append([_regs(ops[0]), 0, i])


def scan_function(text):
    """Hazards in one function's assembly: a list of (line, message)."""
    lines = text.split("\n")
    at_label, found = {}, []
    _scan(lines, at_label, lambda i, m: None)  # first pass: collect branch targets
    _scan(lines, at_label, lambda i, m: found.append((i + 1, m)))
    return found


def split_kernels(asm, pattern):
    """{symbol: body} of every kernel whose symbol matches `pattern`."""
    out = {}
    for m in re.finditer(r"^(" + pattern + r"):[^\n]*\n(.*?)s_endpgm", asm, re.S | re.M):
        out[m.group(1)] = m.group(2) + "s_endpgm\n"
    return out
