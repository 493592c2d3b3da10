"""Inline asm in the device sources declares the scalar state it changes.

An asm statement is opaque to the compiler: if its text writes SCC (any SALU
arithmetic, logic, shift or compare) or M0 without naming them among the
clobbers, the scheduler may place a compare before the statement and the
select that reads SCC after it, and the select then sees the asm's carry.
Host-only check over every file under csrc/.
"""
import glob
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "dense_fp16_gemm_hgemm_amd", "csrc")

# SALU instructions that write SCC (or, for s_cselect / s_cmov, read it)
SCC_OPS = re.compile(
    r"\bs_(add|addc|sub|subb|and|or|xor|andn2|orn2|nand|nor|xnor|lshl|lshr|ashr|bfe|bfm|"
    r"cmp|cmpk|bitcmp0|bitcmp1|min|max|abs|absdiff|not|bcnt0|bcnt1|cselect|cmov|addk|mulk)\w*")
M0_WRITE = re.compile(r"\bs_\w+\s+m0\b")


def asm_statements(text):
    """(template, clobbers) of every `asm [volatile] (...)` statement in C++ source text."""
    out = []
    for m in re.finditer(r"\basm\s+(?:volatile\s*)?\(", text):
        i, depth, parts, cur = m.end(), 1, [], []
        while depth:
            c = text[i]
            if c == '"':
                j = i + 1
                while text[j] != '"':
                    j += 2 if text[j] == "\\" else 1
                cur.append(text[i:j + 1])
                i = j + 1
                continue
            if c == "(":
                depth += 1
            elif c == ")":
                depth -= 1
            elif c == ":" and depth == 1:
                parts.append(cur)
                cur = []
            i += 1
        parts.append(cur)
        strings = [[s[1:-1] for s in p] for p in parts]
        template = "".join(strings[0])
        clobbers = strings[3] if len(strings) > 3 else []
        out.append((template, clobbers))
    return out


def undeclared(template, clobbers):
    missing = []
    if SCC_OPS.search(template) and "scc" not in clobbers:
        missing.append("scc")
    if M0_WRITE.search(template) and "m0" not in clobbers:
        missing.append("m0")
    return missing


def test_the_checker_finds_a_planted_scc_write():
    bad = ('asm volatile("s_add_u32 m0, %0, %1\\n\\tbuffer_load_dwordx4 %2, %3, %4 offen lds"'
           ' : : "s"(a), "n"(8), "v"(v), "s"(r), "s"(k) : "memory", "m0");')
    good = bad.replace('"memory", "m0"', '"memory", "m0", "scc"')
    movm0 = ('asm volatile("s_mov_b32 m0, %0\\n\\tbuffer_load_dword %1, %2, %3 offen lds"'
             ' : : "s"(a), "v"(v), "s"(r), "s"(k) : "memory");')
    (t, c), = asm_statements(bad)
    assert undeclared(t, c) == ["scc"]
    (t, c), = asm_statements(good)
    assert undeclared(t, c) == []
    (t, c), = asm_statements(movm0)
    assert undeclared(t, c) == ["m0"]


def test_device_asm_declares_scc_and_m0():
    files = sorted(glob.glob(os.path.join(CSRC, "*.hpp")) + glob.glob(os.path.join(CSRC, "*.hip")) +
                   glob.glob(os.path.join(CSRC, "*.h")))
    assert files
    seen, bad = 0, []
    for path in files:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        for template, clobbers in asm_statements(text):
            seen += 1
            missing = undeclared(template, clobbers)
            if missing:
                bad.append((os.path.basename(path), template[:60], missing))
    assert seen > 0
    assert not bad, bad
