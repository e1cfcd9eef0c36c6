"""Hazards around the kernels' inline-asm tile copies, checked in the compiled
code (CPU only: each translation unit is compiled to gfx950 assembly here with
the library's own flags).

The compiler inserts the wait states and keeps SCC safe for the instructions
it generates, but an asm block is opaque to it. Two rules of the gfx9-family
ISA's hazard table matter to the copies' blocks (`buffer_load ... lds`):

* an SGPR written by a VALU instruction (readfirstlane, a compare, a carry
  out) and then read by a vector-memory instruction needs 5 wait states in
  between; the copy reads its buffer resource (4 SGPRs) that way;
* an asm block that sets SCC must not sit between an SCC writer and its
  reader (the source-level check is in test_asm_lint.py; this one looks at
  the generated code).
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from long_context_causal_amd import build as gbuild

CSRC = gbuild.CSRC
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
VMEM_SGPR_WAIT_STATES = 5
# VALU opcodes whose second operand is an SGPR destination (carry or condition out)
CARRY_OUT = ("v_add_co_", "v_sub_co_", "v_subrev_co_", "v_addc_co_", "v_subb_co_", "v_subbrev_co_",
             "v_mad_u64_u32", "v_mad_i64_i32", "v_div_scale_")
SCC_READERS = ("s_addc_u32", "s_subb_u32", "s_cselect_", "s_cbranch_scc", "s_cmovk_", "s_cmov_")
SCC_NEUTRAL = ("s_mov_", "s_movk_", "s_nop", "s_waitcnt", "s_barrier", "s_setprio", "s_sleep", "s_cselect_",
               "s_cbranch_", "s_branch", "s_memtime", "s_memrealtime", "s_getreg_", "s_sendmsg", "s_dcache_",
               "s_icache_", "s_endpgm", "s_trap", "s_load_", "s_buffer_load_")


def sgprs(tok):
    tok = tok.strip()
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def operands(line):
    parts = line.split(None, 1)
    return [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []


def valu_sgpr_defs(line):
    op = line.split()[0]
    if not op.startswith("v_"):
        return set()
    ops = operands(line)
    out = set()
    if ops and (op.startswith(("v_readfirstlane", "v_readlane", "v_cmp_", "v_cmp_class")) or op.endswith("_e64")):
        out |= sgprs(ops[0])
    if len(ops) > 1 and op.startswith(CARRY_OUT):
        out |= sgprs(ops[1])
    return out


def instructions(text):
    return [l.strip() for l in text.splitlines()
            if l.strip() and not l.strip().startswith((";", ".")) and not l.strip().endswith(":")]


def copy_hazards(text):
    """(copies seen, list of violations) for the VALU-SGPR -> copy rule."""
    ins = instructions(text)
    bad, n = [], 0
    for k, line in enumerate(ins):
        if not (line.startswith("buffer_load") and line.endswith(" lds")):
            continue
        n += 1
        read = set()  # the resource and the SGPR offset (the operands' SGPRs)
        for o in operands(line):
            read |= sgprs(o.split()[0] if o else o)
        waits = 0
        for j in range(k - 1, -1, -1):
            if waits >= VMEM_SGPR_WAIT_STATES:
                break
            prev = ins[j]
            if valu_sgpr_defs(prev) & read:
                bad.append("%s  ...(%d wait states)...  %s" % (prev, waits, line))
                break
            op = prev.split()[0]
            waits += int(operands(prev)[0]) + 1 if op == "s_nop" else 1
    return n, bad


def scc_hazards(text):
    lines = [l.strip() for l in text.splitlines()]
    bad, k = [], 0
    while k < len(lines):
        if lines[k].startswith(";;#ASMSTART"):
            j = k + 1
            body = []
            while not lines[j].startswith(";;#ASMEND"):
                body.append(lines[j])
                j += 1
            writes = [b.split()[0] for b in body if b.startswith("s_") and not b.startswith(SCC_NEUTRAL)]
            if writes:
                for m in range(j + 1, len(lines)):
                    t = lines[m]
                    if not t or t.startswith((";", ".")) or t.endswith(":"):
                        continue
                    op = t.split()[0]
                    if op.startswith(SCC_READERS):
                        bad.append("asm %s then %s" % (writes, t))
                        break
                    if op.startswith("s_") and not op.startswith(SCC_NEUTRAL):
                        break
            k = j
        k += 1
    return bad


def test_scanner_finds_planted_hazards():
    planted = """
\tv_readfirstlane_b32 s42, v1
\ts_mov_b32 s43, s11
\t;;#ASMSTART
\ts_mov_b32 m0, s1
\ts_nop 0
\tbuffer_load_dword v66, s[40:43], 0 offen lds
\t;;#ASMEND
"""
    n, bad = copy_hazards(planted)
    assert n == 1 and len(bad) == 1
    safe = planted.replace("s_nop 0", "s_nop 3")
    assert copy_hazards(safe) == (1, [])
    carry = planted.replace("v_readfirstlane_b32 s42, v1", "v_add_co_u32_e64 v3, s[42:43], v1, v2")
    assert len(copy_hazards(carry)[1]) == 1
    scc = """
\ts_add_u32 s68, s59, s64
\t;;#ASMSTART
\ts_add_u32 m0, s63, 0
\ts_nop 0
\tbuffer_load_dwordx4 v177, s[4:7], 0 offen lds
\t;;#ASMEND
\ts_addc_u32 s69, s60, s65
"""
    assert len(scc_hazards(scc)) == 1
    assert scc_hazards(scc.replace("s_addc_u32 s69, s60, s65", "s_add_u32 s69, s60, s65")) == []


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not found")
@pytest.mark.parametrize("unit", sorted(gbuild.UNITS))
def test_compiled_copies_have_no_hazard(unit):
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, unit + ".s")
        flags = [f for f in gbuild.COMMON_FLAGS if f not in ("-Wall",)] + gbuild.UNITS[unit]
        cmd = [HIPCC] + flags + ["-I", os.path.join(os.path.dirname(CSRC), "..", "include"), "-I", CSRC,
                                 "--cuda-device-only", "-S", os.path.join(CSRC, unit), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text = open(out).read()
    n, bad = copy_hazards(text)
    assert not bad, "%s: %d copies, VALU-written SGPR read too soon:\n%s" % (unit, n, "\n".join(bad[:5]))
    scc = scc_hazards(text)
    assert not scc, "%s: SCC live across an asm block:\n%s" % (unit, "\n".join(scc[:5]))
    if unit != "gqa_attn.hip":
        assert n > 0  # every kernel unit copies tiles
