"""Rules the kernel sources must keep, checked on the CPU.

A vector store written in inline asm is invisible to the compiler's hazard
recognizer, which leaves wait states after its own 16-byte stores before a
VALU write of the stored registers but none after an asm store; without them
a kernel with several stores per wave stored wrong values.  Every asm
statement in the kernel sources that issues a global or buffer store must
therefore carry an s_nop in the same statement."""

import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_kv_cache_slot_amd", "csrc")

ASM = re.compile(r"__asm__\s+volatile\s*\((.*?)\)\s*;", re.S)
STRING = re.compile(r'"((?:[^"\\]|\\.)*)"')


def _asm_texts(path):
    with open(path) as f:
        src = f.read()
    for m in ASM.finditer(src):
        # the instruction text: the string literals before the first ':'
        head = m.group(1).split(":", 1)[0]
        yield "".join(STRING.findall(head))


def test_asm_stores_carry_their_wait_states():
    files = glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp"))
    assert files
    stores = 0
    for path in files:
        for text in _asm_texts(path):
            if re.search(r"\b(global|buffer)_store", text):
                stores += 1
                assert re.search(r"s_nop\s+[2-9]", text), (
                    f"{os.path.basename(path)}: asm store without wait states: {text!r}")
    assert stores >= 1   # the store helper exists and was found


def test_rule_catches_a_store_without_wait_states(tmp_path):
    bad = tmp_path / "bad.hip"
    bad.write_text('__asm__ volatile("global_store_dwordx4 %0, %1, off nt" : : "v"(p), "v"(v));\n')
    texts = list(_asm_texts(str(bad)))
    assert texts and not re.search(r"s_nop\s+[2-9]", texts[0])
