"""Check the gfx950 assembly of libkvarn for MFMA operand aliasing.

An MFMA whose destination registers overlap its A or B source registers computes
wrong results on gfx950 (rows read after the first pass see the partial output).
The compiler may allocate such a destination when a source dies at that MFMA; the
kernels keep their sources alive, and this check verifies it on the generated code.

Usage: python -m kv_cache_bit_amd.isa_check   (compiles with --save-temps into a temp dir)
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

from . import build as B

REG = re.compile(r"([va])\[(\d+):(\d+)\]|([va])(\d+)")


def _ranges(ops: str):
    out = []
    for m in REG.finditer(ops):
        if m.group(1):
            out.append((m.group(1), int(m.group(2)), int(m.group(3))))
        else:
            out.append((m.group(4), int(m.group(5)), int(m.group(5))))
    return out


def check_asm(text: str) -> list[str]:
    bad = []
    fn = "?"
    for line in text.splitlines():
        s = line.strip()
        if s.endswith(":") and not s.startswith("."):
            fn = s[:-1]
        if not s.startswith("v_mfma"):
            continue
        ops = s.split(None, 1)[1].split(";")[0]
        regs = _ranges(ops)
        if len(regs) < 3:
            continue
        d, a, b = regs[0], regs[1], regs[2]
        for src in (a, b):
            if src[0] == d[0] and not (src[2] < d[1] or d[2] < src[1]):
                bad.append(f"{fn}: {s}")
    return bad


def main() -> int:
    bad = []
    # the library and its butterfly-rotation build (libkvarn_fwht.so)
    for defines in ((), ("-DKVARN_ROTATION_BUTTERFLY=1",)):
        with tempfile.TemporaryDirectory() as tmp:
            for src in B.SOURCES:
                cmd = [B.hipcc(), *[f for f in B.FLAGS if f != "-shared"], *defines, "-c",
                       os.path.join(B.CSRC, src), "-o", os.path.join(tmp, src + ".o"), "--save-temps"]
                subprocess.run(cmd, cwd=tmp, check=True, capture_output=True)
                for f in os.listdir(tmp):
                    if f.endswith(".s") and "gfx950" in f and f.startswith(src.split(".")[0]):
                        bad += check_asm(open(os.path.join(tmp, f)).read())
    for b in bad:
        print("MFMA destination overlaps a source:", b)
    print("isa_check:", "FAIL" if bad else "ok")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
