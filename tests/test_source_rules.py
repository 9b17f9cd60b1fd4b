"""Rules the sources keep, checked on the CPU.

Inline asm: the compiler inserts the wait states a VALU instruction needs after a matrix-core,
transcendental or cross-lane result only for instructions it can see, so inline asm in the
kernels is limited to LDS accesses (which wait for their own results), explicit waits, and
v_bfi_b32 (whose operands are LDS data or plain VALU results).  A max written as asm once read
score-MFMA accumulators before they were written.

bench.py measures one GPU: asked for more, it exits with a message before touching a device.
"""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_encode_amd", "csrc")
ALLOWED = re.compile(r"^(ds_\w+|s_waitcnt|s_nop|v_bfi_b32)$")


def asm_mnemonics(text):
    """Mnemonics of every instruction in the string literals of asm statements."""
    out = []
    for m in re.finditer(r"\basm\s*(?:volatile\s*)?\(", text):
        i, depth = m.end(), 1
        while depth and i < len(text):
            depth += {"(": 1, ")": -1}.get(text[i], 0)
            i += 1
        body = text[m.end():i - 1]
        # the template: the string literals at the start of the statement, before the first
        # operand colon (colons inside the strings, as in offset0:1, belong to the template)
        lits = re.match(r'\s*((?:"(?:[^"\\]|\\.)*"\s*)+)', body)
        literal = "".join(re.findall(r'"((?:[^"\\]|\\.)*)"', lits.group(1))) if lits else ""
        for ins in literal.replace("\\n", "\n").replace("\\t", " ").split("\n"):
            ins = ins.strip()
            if ins:
                out.append(ins.split()[0])
    return out


def test_inline_asm_is_limited_to_lds_waits_and_bfi():
    seen = []
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            text = open(os.path.join(CSRC, name)).read()
            text = re.sub(r"//[^\n]*", "", text)
            for mn in asm_mnemonics(text):
                seen.append(mn)
                assert ALLOWED.match(mn), f"{name}: inline asm instruction {mn} is not in the allowed set"
    assert any(m.startswith("ds_read") for m in seen)  # the scan found the kernels' asm


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
