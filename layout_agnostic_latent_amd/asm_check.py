"""Build-time check of the decode kernel's gfx950 assembly: no instruction may
touch the accumulator of a score-MFMA chain while its result is in flight.

The score MFMAs are issued from inline asm (VGPR accumulators beside the AGPR
output tiles).  The compiler takes an asm statement's output as written when
the statement issues, while the matrix core writes it several passes later,
and its hazard recognizer cannot see into the asm.  Chained MFMAs that
accumulate into the same registers need no wait states, so between two MFMAs
of a chain nothing else may read or write the accumulator (a register-
allocator copy there would read stale values), and after the chain's last
MFMA nothing may until enough wait states have passed (the last statement of
a chain carries them itself).

Usage: ``python -m layout_agnostic_latent_amd.asm_check`` (compiles
``csrc/decode_attn.hip`` to assembly with the library's flags and scans it).
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

from layout_agnostic_latent_amd import build as _build

# wait states a VALU read of a 32x32x16 MFMA result needs on gfx950 (the
# kernel's chain ends with s_nop 7, 7, 3 = 20)
_MIN_WAITS = 18
_MFMA = re.compile(r"v_mfma_\w+\s+([va]\[\d+:\d+\])")
_REG = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")


def _regs(text: str) -> set:
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            out.update((m.group(3), r) for r in range(int(m.group(4)), int(m.group(5)) + 1))
    return out


def scan(asm_text: str) -> list:
    """Return (line number, message) for every access to an in-flight chain accumulator.

    Each chain's accumulator (the VGPR result of an inline-asm MFMA) is in
    flight until _MIN_WAITS wait states have issued after its last MFMA:
    every instruction counts as one, an s_nop N as N + 1.  Only the next MFMA
    of the same chain may touch it earlier.  A label or a branch inside that
    window is reported too: the wait states counted along the straight-line
    code would not hold on another path.
    """
    bad = []
    in_asm = False
    pending = {}  # accumulator registers -> [line index of its last MFMA, wait states since]

    def flush(i, why):
        for regs, (line, _) in list(pending.items()):
            bad.append((i + 1, f"{why} inside the wait window of the accumulator written at line {line + 1}"))
        pending.clear()

    def tick(i, t, op, regs, n):
        for key, st in list(pending.items()):
            if regs & key:
                bad.append((i + 1, f"accesses the in-flight accumulator of line {st[0] + 1}: {t}"))
                del pending[key]
                continue
            st[1] += n
            if st[1] >= _MIN_WAITS:
                del pending[key]

    for i, line in enumerate(asm_text.split("\n")):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if re.match(r"^[.\w]+:", t):  # a label: another path may enter here
            if pending:
                flush(i, "label")
            continue
        if not t or t.startswith(";") or t.startswith("."):
            continue
        op = t.split()[0]
        if op.startswith("s_cbranch") or op.startswith("s_branch") or op.startswith("s_setpc"):
            if pending:
                flush(i, "branch")
            continue
        regs = _regs(t)
        if op.startswith("v_mfma"):
            m = _MFMA.match(t)
            dst = frozenset(_regs(m.group(1))) if m else frozenset()
            if dst in pending:
                del pending[dst]  # the chain continues: back-to-back accumulation is safe
            tick(i, t, op, regs, 1)
            if in_asm and m and m.group(1).startswith("v"):
                pending[dst] = [i, 0]
            continue
        tick(i, t, op, regs, int(t.split()[1]) + 1 if op == "s_nop" else 1)
    return bad


def compile_asm(src: str = "decode_attn.hip") -> str:
    """gfx950 device assembly of one library source, with the library's own flags."""
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [_build.hipcc()] + _build.compile_flags() + ["--cuda-device-only", "-S",
                                                           os.path.join(_build.CSRC, src), "-o", out]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"assembly build failed: {' '.join(cmd)}\n{r.stdout}")
        return open(out).read()


def main() -> int:
    text = compile_asm()
    n_chain = sum(1 for l in text.split("\n") if "v_mfma" in l and ("v[2:17]" in l or "v[18:33]" in l))
    bad = scan(text)
    for ln, msg in bad:
        print(f"decode_attn.s:{ln}: {msg}")
    print(f"{n_chain} score-chain MFMAs scanned, {len(bad)} violations")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
