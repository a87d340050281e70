"""Hazard check for the MFMAs written as inline assembly (build-time tool).

The compiler inserts the wait states that gfx950 requires around the MFMAs it
emits itself, but an MFMA inside an inline-assembly statement is opaque to it.
The wide prefill kernel issues its score MFMAs that way (to fix their
register classes), so two hazards are the source's responsibility:

  * a VALU instruction (including the compiler's own AGPR<->VGPR moves)
    writing a register that an inline-assembly MFMA reads within the next
    `before` wait states (the hardware needs 2);
  * an instruction other than an MFMA reading an inline-assembly MFMA's
    result registers within `after` wait states of it (a 32x32x16 result
    needs up to 18).

check_asm() scans gfx950 assembly for both and returns the offending pairs;
compile_to_asm() produces that assembly for one source file.

    python -m exact_attention_17_amd.isa_check      # checks prefill_wide.hip
"""

import os
import re
import subprocess
import sys
import tempfile

from .build import ARCH, CSRC, INCLUDE, hipcc_path

_RANGE = re.compile(r"([va])\[(\d+):(\d+)\]$")
_SINGLE = re.compile(r"([va])(\d+)$")


def _regs(tok):
    """Register names covered by one operand token (v7, a[4:7], ...)."""
    m = _RANGE.match(tok)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {tok} if _SINGLE.match(tok) else set()


def _instructions(text):
    """(opcode, operands, from_inline_asm) for every instruction in the text."""
    out, in_asm = [], False
    for line in text.splitlines():
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        s = s.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        parts = s.replace(",", " ").split()
        out.append((parts[0], parts[1:], in_asm))
    return out


def _wait_states(op, args):
    return int(args[0]) + 1 if op == "s_nop" else 1


def check_asm(text, before=3, after=19):
    """Hazards of inline-assembly MFMAs in `text`; an empty list means none."""
    insts = _instructions(text)
    found = []
    for i, (op, args, asm) in enumerate(insts):
        if not (asm and op.startswith("v_mfma")):
            continue
        srcs = set().union(*(_regs(a) for a in args[1:4]))
        k, ws = i - 1, 0
        while k >= 0 and ws < before:
            op2, args2, _ = insts[k]
            if op2.startswith("v_") and not op2.startswith("v_mfma") and args2:
                if _regs(args2[0]) & srcs:
                    found.append(f"{op2} {args2[0]} written {ws} wait states before {op} {' '.join(args)}")
            ws += _wait_states(op2, args2)
            k -= 1
        dst = _regs(args[0])
        k, ws = i + 1, 0
        while k < len(insts) and ws < after:
            op2, args2, _ = insts[k]
            if op2 in ("s_branch", "s_endpgm") or op2.startswith("s_cbranch"):
                break
            if not op2.startswith("v_mfma"):
                read = set()
                first = 1 if op2.startswith(("v_", "ds_read", "buffer_load", "global_load")) else 0
                for a in args2[first:]:
                    read |= _regs(a)
                if read & dst:
                    found.append(f"{op2} {' '.join(args2)} reads {op} {args[0]} after {ws} wait states")
            ws += _wait_states(op2, args2)
            k += 1
    return found


_SGPR_RANGE = re.compile(r"s\[(\d+):(\d+)\]$")
_SGPR = re.compile(r"s(\d+)$")


def _sregs(tok):
    """SGPR names covered by one operand token (s7, s[4:7], m0)."""
    m = _SGPR_RANGE.match(tok)
    if m:
        return {f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    if _SGPR.match(tok) or tok == "m0":
        return {tok}
    return set()


def check_lds_loads(text, valu_sgpr=5, m0=1):
    """Hazards of inline-assembly direct-to-LDS buffer loads in `text`: a VALU
    instruction (v_readfirstlane and the like) writing one of the load's SGPR
    operands within `valu_sgpr` wait states before it, or an M0 write within
    `m0` wait states before it.  An empty list means none."""
    insts = _instructions(text)
    found = []
    for i, (op, args, asm) in enumerate(insts):
        if not (asm and op.startswith("buffer_load") and "lds" in args):
            continue
        sg = set().union(*(_sregs(a) for a in args[1:4]))
        k, ws = i - 1, 0
        while k >= 0 and ws < max(valu_sgpr, m0):
            op2, args2, _ = insts[k]
            if op2.startswith(("s_branch", "s_cbranch")) or op2.endswith(":"):
                break
            dst = _sregs(args2[0]) if args2 else set()
            if op2.startswith("v_") and ws < valu_sgpr and dst & sg:
                found.append(f"{op2} {args2[0]} written {ws} wait states before {op} {' '.join(args)}")
            if "m0" in dst and ws < m0:
                found.append(f"{op2} m0 written {ws} wait states before {op} {' '.join(args)}")
            ws += _wait_states(op2, args2)
            k -= 1
    return found


def compile_to_asm(source="prefill_wide.hip"):
    """gfx950 assembly of one source file, compiled as the library is."""
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "out.s")
        cmd = [hipcc_path(), f"--offload-arch={ARCH}", "-O3", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument", "--cuda-device-only", "-S",
               "-I", INCLUDE, "-I", CSRC, "-o", out, os.path.join(CSRC, source)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-4000:]}")
        return open(out).read()


if __name__ == "__main__":
    text = compile_to_asm(*(sys.argv[1:2] or []))
    problems = check_asm(text) + check_lds_loads(text)
    print("\n".join(problems) or "no inline-asm MFMA hazards")
    sys.exit(1 if problems else 0)
