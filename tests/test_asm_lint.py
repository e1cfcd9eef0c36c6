"""Source checks of the kernels' inline asm (CPU only, no build).

The compiler knows nothing of what an asm block does beyond its operands and
clobbers. A scalar ALU instruction that sets SCC (an add's carry, a
compare's result) inside a block that does not list "scc" lets the compiler
keep its own SCC value live across the block, for instance between the two
halves of a 64-bit address add, and the high half then takes the block's
carry. This test finds every asm statement under csrc/ whose template holds
such an instruction and checks its clobber list.
"""
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_causal_amd", "csrc")

# scalar instructions that leave SCC alone (moves, waits, barriers, branches,
# and the selects and conditional branches that only read it)
SCC_NEUTRAL = ("s_mov_", "s_movk_", "s_nop", "s_waitcnt", "s_barrier", "s_setprio", "s_sleep", "s_cselect_",
               "s_cbranch_", "s_branch", "s_memtime", "s_memrealtime", "s_getreg_", "s_sendmsg", "s_dcache_",
               "s_icache_", "s_endpgm", "s_trap", "s_load_", "s_buffer_load_")


def asm_statements(text):
    """(template, clobbers) of every asm statement: the string literals before
    the first ':' are the template, the literals after the third ':' the
    clobbers."""
    out = []
    for m in re.finditer(r"\basm\s+(?:volatile\s*)?\(", text):
        depth, i = 1, m.end()
        while depth:
            c = text[i]
            if c == '"':
                i = text.index('"', i + 1)
                while text[i - 1] == "\\":
                    i = text.index('"', i + 1)
            elif c == "(":
                depth += 1
            elif c == ")":
                depth -= 1
            i += 1
        body = text[m.end():i - 1]
        # split on top-level ':' outside string literals and parentheses
        parts, cur, d, j = [], "", 0, 0
        while j < len(body):
            c = body[j]
            if c == '"':
                k = body.index('"', j + 1)
                while body[k - 1] == "\\":
                    k = body.index('"', k + 1)
                cur += body[j:k + 1]
                j = k + 1
                continue
            if c in "([":
                d += 1
            elif c in ")]":
                d -= 1
            if c == ":" and d == 0:
                parts.append(cur)
                cur = ""
            else:
                cur += c
            j += 1
        parts.append(cur)
        template = "".join(re.findall(r'"((?:[^"\\]|\\.)*)"', parts[0]))
        clobbers = re.findall(r'"([^"]*)"', parts[3]) if len(parts) > 3 else []
        out.append((template, clobbers))
    return out


def scc_writers(template):
    ops = re.findall(r"(?:^|\\n|\\t|;)\s*(s_[a-z0-9_]+)", template)
    return [o for o in ops if not o.startswith(SCC_NEUTRAL)]


def test_parser_finds_the_clobbers():
    text = 'asm volatile("s_add_u32 m0, %0, %1\\n\\ts_nop 0" :: "s"(a), "i"(4) : "memory", "scc");'
    [(template, clobbers)] = asm_statements(text)
    assert scc_writers(template) == ["s_add_u32"]
    assert clobbers == ["memory", "scc"]
    [(template, clobbers)] = asm_statements('asm volatile("s_mov_b32 m0, %0" :: "s"(a));')
    assert scc_writers(template) == [] and clobbers == []


def test_scc_writing_asm_declares_the_clobber():
    files = sorted(glob.glob(os.path.join(CSRC, "*.hpp")) + glob.glob(os.path.join(CSRC, "*.hip")))
    assert files
    seen = 0
    for path in files:
        for template, clobbers in asm_statements(open(path).read()):
            w = scc_writers(template)
            if w:
                seen += 1
                assert "scc" in clobbers, "%s: asm with %s lacks the scc clobber" % (os.path.basename(path), w)
    assert seen >= 1  # the tile copies' M0 add
