"""Check the gfx950 assembly of libkvarn for MFMA operand aliasing, scratch and calls.

An MFMA whose destination registers overlap its A or B source registers computes
wrong results on gfx950 (rows read after the first pass see the partial output).
The compiler may allocate such a destination when a source dies at that MFMA; the
kernels keep their sources alive, and this check verifies it on the generated code.
It also refuses any function that uses scratch memory or calls another: the kernels
keep their state in registers and LDS.

Usage: python -m kv_cache_bit_amd.isa_check   (compiles the device code to assembly in a temp dir)
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


def check_resources(text: str) -> list[str]:
    """Functions of the generated code that use scratch memory or call other functions:
    every kernel of the library keeps its state in registers and LDS (a device function
    called for real passes its arrays through scratch, at a heavy cost per tile)."""
    bad = []
    fn = "?"
    for line in text.splitlines():
        s = line.strip()
        if s.endswith(":") and not s.startswith(".") and not s.startswith(";"):
            fn = s[:-1]
        if s.startswith("s_swappc") or s.startswith("s_setpc"):
            bad.append(f"{fn}: call ({s.split()[0]})")
        if s.startswith("; ScratchSize:") and s.split(":")[1].strip() not in ("0", "0 bytes/lane"):
            bad.append(f"{fn}: {s[2:]}")
    return bad


def device_asm(src: str, defines: tuple, tmp: str) -> str:
    """The gfx950 assembly of one source, as the library build compiles it."""
    out = os.path.join(tmp, src + ".s")
    cmd = [B.hipcc(), *[f for f in B.FLAGS if f != "-shared"], *defines, "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return f.read()


def main() -> int:
    from concurrent.futures import ThreadPoolExecutor
    # the library and its butterfly-rotation build (libkvarn_fwht.so), one hipcc per source
    variants = ((), ("-DKVARN_ROTATION_BUTTERFLY=1",))
    with tempfile.TemporaryDirectory() as tmp, ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        jobs = []
        for i, defines in enumerate(variants):
            d = os.path.join(tmp, str(i))
            os.makedirs(d)
            jobs += [ex.submit(device_asm, src, defines, d) for src in B.SOURCES]
        texts = [j.result() for j in jobs]
    if sum(t.count("v_mfma") for t in texts) == 0:
        print("isa_check: no MFMA found in the generated code")
        return 1
    bad = [b for t in texts for b in check_asm(t)]
    for b in bad:
        print("MFMA destination overlaps a source:", b)
    res = [b for t in texts for b in check_resources(t)]
    for b in res:
        print("scratch memory or a call:", b)
    bad += res
    print("isa_check:", "FAIL" if bad else "ok")
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
