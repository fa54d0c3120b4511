"""The wide buffer stores of the HIP sources keep soffset = 0.

A 16-byte buffer store of the multi-token decode once carried its row-block
offset in a register soffset; the compiler then let the next VALU instruction
overwrite the store's last data register before the store had read it, and
the last dword of some stores held the new value.  With soffset = 0 and the
offset in the lane's voffset the compiler keeps the data registers intact.
Every wide (8, 12 or 16-byte) buffer store in the library follows that
convention; this test fails on any that does not, written through the
builtins or through inline assembly."""
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = sorted(glob.glob(os.path.join(ROOT, "gated_delta_rule_23_amd", "csrc", "*.hip"))
                 + glob.glob(os.path.join(ROOT, "gated_delta_rule_23_amd", "csrc", "*.h"))
                 + glob.glob(os.path.join(ROOT, "gated_delta_rule_23_amd", "csrc", "*.cpp")))

WIDE_BUILTIN = re.compile(r"__builtin_amdgcn_raw(?:_ptr)?_buffer_store_(b64|b96|b128)\s*\(")
WIDE_ASM = re.compile(r"buffer_store_dwordx(2|3|4)\b([^\"\\]*)")


def strip_comments(text):
    text = re.sub(r"/\*.*?\*/", lambda m: " " * len(m.group(0)), text, flags=re.S)
    return re.sub(r"//[^\n]*", "", text)


def call_args(text, start):
    """The top-level comma-separated arguments of the call whose '(' is at
    text[start - 1]."""
    depth, args, cur, i = 1, [], [], start
    while i < len(text) and depth:
        c = text[i]
        if c in "([{":
            depth += 1
        elif c in ")]}":
            depth -= 1
            if depth == 0:
                break
        if c == "," and depth == 1:
            args.append("".join(cur).strip())
            cur = []
        else:
            cur.append(c)
        i += 1
    args.append("".join(cur).strip())
    return args


def wide_store_soffsets(text):
    """(line, soffset text) of every wide buffer store in a source text."""
    text = strip_comments(text)
    out = []
    for m in WIDE_BUILTIN.finditer(text):
        args = call_args(text, m.end())
        # (data, rsrc, voffset, soffset, aux)
        out.append((text.count("\n", 0, m.start()) + 1, args[3] if len(args) == 5 else "<unparsed>"))
    for m in WIDE_ASM.finditer(text):
        ops = [o.strip() for o in m.group(2).split(",")]
        # buffer_store_dwordxN vdata, vaddr, srsrc, soffset [offen ...]
        soff = ops[3].split()[0] if len(ops) > 3 and ops[3] else "<unparsed>"
        out.append((text.count("\n", 0, m.start()) + 1, soff))
    return out


def test_parser_sees_register_soffsets():
    """The scanner itself: a literal 0 passes, anything else is reported."""
    src = """
      __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);   // ok
      __builtin_amdgcn_raw_buffer_store_b64(f(a, b), r, x + 4, soff, 0);
      /* __builtin_amdgcn_raw_buffer_store_b128(v, r, off, s, 0); in a comment */
      asm volatile("buffer_store_dwordx4 %0, %1, %2, %3 offen" :: "v"(d), "v"(o), "s"(r), "s"(s));
      asm volatile("buffer_store_dwordx2 %0, %1, %2, 0 offen" :: "v"(d), "v"(o), "s"(r));
      __builtin_amdgcn_raw_buffer_store_b32(v, r, off, s, 0);   // 4 bytes: not a wide store
    """
    found = wide_store_soffsets(src)
    assert [s for _, s in found] == ["0", "soff", "%3", "0"]


@pytest.mark.parametrize("path", SOURCES, ids=os.path.basename)
def test_wide_buffer_stores_use_a_zero_soffset(path):
    with open(path, encoding="utf-8") as f:
        found = wide_store_soffsets(f.read())
    bad = [(line, s) for line, s in found if s != "0"]
    assert not bad, f"{os.path.basename(path)}: wide buffer stores with soffset != 0 at lines {bad}"


def test_the_library_has_wide_stores_to_check():
    total = 0
    for p in SOURCES:
        with open(p, encoding="utf-8") as f:
            total += len(wide_store_soffsets(f.read()))
    assert total >= 3
