"""Static check of the inline-asm MFMAs in AMD GPU assembly (test infrastructure).

The compiler inserts the wait states an MFMA needs only around MFMAs it knows about; inline
asm is opaque to it.  For every MFMA inside an inline-asm region of one kernel this reports
  PRE:  a non-MFMA, non-memory instruction writing one of its source registers less than
        `pre` wait states before it;
  POST: a non-MFMA instruction reading or writing its destination less than `post` wait
        states after it;
scanning the instructions in program order (across block labels, which over-approximates
the paths).  `s_nop N` counts N + 1 wait states, every other instruction 1; a scan for a
register stops at its next redefinition by another instruction."""
import re

MEMORY = ("ds_", "global_load", "buffer_load", "scratch_load", "flat_load")
STORES = ("global_store", "buffer_store", "scratch_store", "ds_write", "flat_store")


def _regs(tok):
    out = set()
    for m in re.finditer(r"([va])\[(\d+):(\d+)\]|([va])(\d+)\b", tok):
        if m.group(1):
            out |= {f"{m.group(1)}{r}" for r in range(int(m.group(2)), int(m.group(3)) + 1)}
        else:
            out.add(f"{m.group(4)}{m.group(5)}")
    return out


def _parse(s):
    op = s.split()[0]
    ops = [x.strip() for x in s[len(op):].split(",")] if len(s) > len(op) else []
    return op, ops


def _wait_states(op, ops):
    return int(ops[0], 0) + 1 if op == "s_nop" else 1


def _body(text, kernel):
    lines = text.split("\n")
    start = next(i for i, l in enumerate(lines) if l.startswith(kernel + ":"))
    end = next(i for i in range(start, len(lines)) if "s_endpgm" in lines[i])
    body, in_asm = [], False
    for l in lines[start + 1:end]:
        s = l.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not s or s.startswith(";") or s.endswith(":"):
            continue
        body.append((s.split(";")[0].strip(), in_asm))
    return body


def check(text, kernel, pre=8, post=24):
    """List of hazard descriptions (empty: none) for `kernel` (its mangled name) in `text`."""
    body = _body(text, kernel)
    issues = []
    for idx, (s, in_asm) in enumerate(body):
        if not in_asm or not s.startswith("v_mfma"):
            continue
        op, ops = _parse(s)
        dst = _regs(ops[0])
        live = set().union(*[_regs(o) for o in ops[1:]])
        w, j = 0, idx - 1
        while j >= 0 and live and w < pre:
            s2 = body[j][0]
            op2, ops2 = _parse(s2)
            wr = _regs(ops2[0]) if ops2 and not op2.startswith(("s_",) + STORES) else set()
            if wr & live and not op2.startswith(MEMORY + ("v_mfma",)):
                issues.append(f"PRE {w}: {s2}  ->  {s}")
            live -= wr
            w += _wait_states(op2, ops2)
            j -= 1
        live, w, j = set(dst), 0, idx + 1
        while j < len(body) and w < post:
            s2 = body[j][0]
            op2, ops2 = _parse(s2)
            if not op2.startswith(("v_mfma", "s_")):
                used = set().union(*[_regs(o) for o in ops2]) if ops2 else set()
                if used & live:
                    issues.append(f"POST {w}: {s}  ->  {s2}")
                    break
            w += _wait_states(op2, ops2)
            j += 1
    return issues
