"""Rules of the HIP sources that the compiler does not enforce, checked on
the text (no GPU):

* the compiler inserts no wait states into inline assembly, so every inline
  copy that reads a scalar base or M0 starts with them: s_nop 4 before a
  vector-memory instruction whose scalar base a vector instruction may have
  just written (5 wait states), at least s_nop 0 before an LDS copy that only
  reads M0 (1 wait state);
* readfirstlane returns a signed int, so a 64-bit value rebuilt from it must
  widen each half as unsigned (readfirstlane_ptr does), or a low word with bit
  31 set sign-extends into the high word.
"""
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "block_draft_head_amd", "csrc")
SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp", ".cpp")))
VMEM = re.compile(r"\b(global_load|global_store|global_atomic|buffer_load|buffer_store|scratch_)\w*")


def asm_blocks(text):
    """(instruction string, operand text) of every asm statement."""
    for m in re.finditer(r"asm\s+volatile\s*\(", text):
        i, depth = m.end(), 1
        while depth:
            depth += {"(": 1, ")": -1}.get(text[i], 0)
            i += 1
        body = text[m.end():i - 1]
        # the template: the string literals before the first operand colon
        strings, j = [], 0
        while True:
            lit = re.match(r'\s*"((?:[^"\\]|\\.)*)"', body[j:])
            if not lit:
                break
            strings.append(lit.group(1))
            j += lit.end()
        yield "".join(strings), body[j:]


def test_sources_are_found():
    names = {os.path.basename(s) for s in SOURCES}
    assert {"lmhead.hip", "proj.hip", "selector.hip", "common.hpp"} <= names


def test_inline_memory_instructions_start_with_their_wait_states():
    checked = 0
    for path in SOURCES:
        text = open(path).read()
        for instr, body in asm_blocks(text):
            lines = [l.strip() for l in instr.replace("\\n", "\n").replace("\\t", "").split("\n") if l.strip()]
            for k, line in enumerate(lines):
                if not VMEM.match(line):
                    continue
                checked += 1
                reads_m0 = "_lds" in line.split()[0]
                scalar_base = re.search(r'"s"\s*\(', body) is not None
                if not (reads_m0 or scalar_base):
                    continue  # vector address only: no wait state needed
                need = 4 if scalar_base else 0
                prev = lines[k - 1] if k else ""
                m = re.match(r"s_nop\s+(\d+)", prev)
                assert m and int(m.group(1)) >= need, (
                    f"{os.path.basename(path)}: '{line}' needs 's_nop {need}' (or more) right before it in the same asm")
    assert checked >= 2


def test_readfirstlane_is_widened_as_unsigned():
    for path in SOURCES:
        for no, line in enumerate(open(path), 1):
            if "__builtin_amdgcn_readfirstlane" not in line:
                continue
            wide = "uint64_t" in line or "<< 32" in line
            assert not wide or "(uint32_t)__builtin_amdgcn_readfirstlane" in line, (
                f"{os.path.basename(path)}:{no}: a readfirstlane result widened to 64 bits must be cast to uint32_t "
                f"first (use readfirstlane_ptr)")
