"""Inline assembly in the HIP sources must not write SCC, the scalar condition code.

The compiler treats SCC as preserved across an inline-asm statement that does
not name it as clobbered, and it does keep carries live across such statements:
a 64-bit scalar address add can be split into its low-word add before a copy
statement and its carry add after it. An SCC-writing instruction inside the
statement (an ``s_add_u32`` into M0, for instance) then drops the carry, and the
copy reads 4 GB away from its tile whenever the low word of the address wraps.
Such a fault depends on where the buffers happen to lie, so passing GPU tests
do not rule it out; this check on the source text does.
"""
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "attention_bga_packed_amd", "csrc")

# scalar ALU and compare instructions that write SCC (gfx9 family)
SCC_WRITERS = re.compile(
    r"^s_(cmp\w*|add_[iu]32|sub_[iu]32|addc_u32|subb_u32|addk_i32|mulk_i32|and_\w+|or_\w+|xor_\w+|andn2_\w+|orn2_\w+|"
    r"nand_\w+|nor_\w+|xnor_\w+|lshl\w*|lshr\w*|ashr\w*|bfe_\w+|min_\w+|max_\w+|abs\w*|not_\w+|bitcmp\w*|bcnt\w*|"
    r"wqm_\w+|quadmask_\w+|absdiff_\w+|cselect_never)\b")

ASM = re.compile(r'asm\s*(?:volatile\s*)?\(\s*((?:"(?:[^"\\]|\\.)*"\s*)+)(.*?)\);', re.S)


def asm_statements(text):
    """(instructions, rest of the statement after the template) for every asm statement in text."""
    out = []
    for m in ASM.finditer(text):
        template = "".join(re.findall(r'"((?:[^"\\]|\\.)*)"', m.group(1)))
        instrs = [i.strip() for i in re.split(r"\\n|;", template.replace("\\t", " ")) if i.strip()]
        out.append((instrs, m.group(2)))
    return out


def scc_violations(text):
    bad = []
    for instrs, rest in asm_statements(text):
        if "scc" in rest:
            continue   # declared clobbered
        for ins in instrs:
            mnemonic = ins.split()[0]
            if SCC_WRITERS.match(mnemonic):
                bad.append(ins)
    return bad


def test_checker_flags_an_scc_writer():
    planted = 'asm volatile("s_add_u32 m0, %2, %3\\n\\ts_nop 0\\n\\tglobal_load_lds_dwordx4 %0, %1" : : "v"(a), "s"(b));'
    assert scc_violations(planted) == ["s_add_u32 m0, %2, %3"]
    clean = 'asm volatile("s_mov_b32 m0, %2\\n\\ts_nop 0\\n\\tglobal_load_lds_dwordx4 %0, %1" : : "v"(a), "s"(b));'
    assert scc_violations(clean) == []
    assert scc_violations('asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));') == []


@pytest.mark.parametrize("name", sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp"))))
def test_no_scc_writes_in_inline_asm(name):
    with open(os.path.join(CSRC, name)) as fh:
        text = fh.read()
    assert scc_violations(text) == [], f"{name}: inline assembly writes SCC without declaring it"
