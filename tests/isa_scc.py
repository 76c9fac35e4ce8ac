"""Scan of gfx950 assembly for a scalar-condition hazard left by the compiler.

A select or conditional branch reads the scalar condition code (SCC). The
instruction that last wrote SCC before it must be the one meant to set the
condition. This scan flags readers (s_cselect, s_cmov, s_cbranch_scc*) whose
nearest earlier SCC writer is a shift, bit-field or min/max instruction, or
any non-compare writer separated from the reader by a branch target. Such an
instruction leaves SCC = (result != 0), almost never the intended condition.

This pattern was found in one build of the head-dim-256 prefill kernel. There
the packed-batch sequence walk computed its work-item values in vector
registers. The compiler placed the select of `nb = len > 0 ? blocks : 0`
after the branch that computes `blocks`, whose scalar arithmetic had
overwritten SCC. `g -= nb` then subtracted 0, and the late query blocks of
every sequence after the first were never computed. The kernels now keep
those values in scalar registers, and no select of this kind remains.
"""
from __future__ import annotations

import re

_SCC_WRITER = re.compile(
    r"^s_(cmp|bitcmp|add|addc|sub|subb|and|or|xor|andn2|orn2|nand|nor|xnor|lshl|lshr|ashr|bfe|"
    r"min|max|abs|not|bcnt|ff|flbit|quadmask|wqm|absdiff|cselect_b64)")
_SUSPECT = re.compile(r"^s_(lshl|lshr|ashr|bfe|min|max|abs|not|bcnt|ff|flbit)")
_READER = re.compile(r"^s_(cselect|cmov|cbranch_scc)")


def suspicious_scc_reads(asm_text: str, window: int = 400):
    """[(line, reader, writer line, writer)] for every flagged SCC reader."""
    lines = [ln.split(";")[0].strip() for ln in asm_text.splitlines()]
    found = []
    for i, ln in enumerate(lines):
        if not _READER.match(ln):
            continue
        crossed_label = False
        for j in range(i - 1, max(-1, i - window), -1):
            p = lines[j]
            if not p:
                continue
            if p.startswith(".LBB") and p.endswith(":"):
                crossed_label = True
                continue
            op = p.split()[0]
            if _SCC_WRITER.match(op):
                if _SUSPECT.match(op) or (crossed_label and not op.startswith(("s_cmp", "s_bitcmp"))):
                    found.append((i + 1, ln, j + 1, p))
                break
    return found
