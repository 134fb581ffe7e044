"""Static VALU instruction mix of a compiled kernel, by issue cost.

Compiles one of the library's HIP sources for gfx950 to assembly (the same
flags as the build) and counts, over the basic blocks given, the vector ALU
instructions of the 2-clock forms (two-operand 32-bit logic, add and shift
on VGPRs with at most a literal or inline constant, i.e. the `_e32`
encodings without an SGPR, VCC, DPP or select operand; and `v_bitop3_b32`
on three VGPRs) and of the 4-clock forms (everything else: 64-bit shifts,
compares and multiply-adds, 32-bit multiplies, 3-input forms, alignbit,
perm, bcnt, DPP, and any form reading an SGPR).  The issue ceiling of the
mix is then peak * 2 / (2 f + 4 (1 - f)) for a fraction f of 2-clock forms,
peak being the 2-clock rate.

    python -m minimizer_sharded_bloom_amd.isa_mix SOURCE KERNEL_SYMBOL [BLOCK,BLOCK,...]

With no block list every block of the kernel counts (the main path of the
query at k=31, m=16, s=28, H=4 is the entry block and the blocks that the
assembly labels for the front end, the records and pass B).
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile
from collections import Counter

from .build import CSRC, common_flags, hipcc


def assemble(src: str) -> str:
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        flags = [f for f in common_flags() if f != "-fPIC"]
        cmd = [hipcc(), "-x", "hip", *flags, "-I" + CSRC, "--cuda-device-only", "-S",
               os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(r.stderr[-2000:])
        return open(out).read()


def two_clock(op: str, args: str) -> bool:
    reads_scalar = re.search(r"\bs\[?\d", args) is not None or "vcc" in args or "exec" in args
    if reads_scalar:
        return False
    if op == "v_bitop3_b32":
        return True
    return op.endswith("_e32") and "dpp" not in op and "cndmask" not in op and "readfirstlane" not in op


def mix(asm: str, symbol: str, blocks=None) -> Counter:
    lines = asm.split("\n")
    start = next(i for i, l in enumerate(lines) if l.startswith(symbol + ":"))
    cur, out = "ENTRY", Counter()
    for line in lines[start + 1:]:
        s = line.strip()
        if s.startswith("s_endpgm"):
            break
        if re.match(r"^\.?[A-Za-z0-9_]+:", s):
            cur = s.split(":")[0]
            continue
        if not s.startswith("v_") or (blocks and cur not in blocks):
            continue
        op = s.split()[0]
        out["2-clock" if two_clock(op, s[len(op):]) else "4-clock"] += 1
    return out


def main() -> None:
    src, symbol = sys.argv[1], sys.argv[2]
    blocks = set(sys.argv[3].split(",")) if len(sys.argv) > 3 else None
    c = mix(assemble(src), symbol, blocks)
    n = c["2-clock"] + c["4-clock"]
    f = c["2-clock"] / n if n else 0.0
    print({"2-clock": c["2-clock"], "4-clock": c["4-clock"], "fraction_2clock": round(f, 3),
           "ceiling_over_2clock_peak": round(2 / (2 * f + 4 * (1 - f)), 3) if n else None})


if __name__ == "__main__":
    main()
