"""Main-loop check of the MFMA kernels' gfx950 assembly.

The forward and input-gradient kernels keep their 256 accumulators in AGPRs and update them
through inline-asm MFMAs, whose result latency the compiler cannot see.  That is only sound
while the compiler never copies an accumulator inside the main loop, and the loop is only fast
while nothing spills to scratch there.  This module compiles a kernel source to device assembly
with the library's own flags and reports, for every kernel instance, the MFMA, scratch and
`v_accvgpr` instruction counts of its main loop (the innermost loop with the most MFMAs).

    python -m qlora_fine_tuning_amd.asm_loops            # fwd.hip and dx.hip
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile

from . import build


def device_asm(source: str) -> str:
    """gfx950 device assembly of one source under csrc/, compiled as the build compiles it."""
    path = os.path.join(build.CSRC, source)
    flags = build.HIP_FLAGS + build.EXTRA_FLAGS.get(source, [])
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        subprocess.run([build._hipcc(), *flags, "-x", "hip", "-S", "--cuda-device-only", path, "-o", out],
                       check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        return open(out).read()


_LABEL = re.compile(r"^(\.LBB\w+):")
_BRANCH = re.compile(r"\bs_(?:cbranch\w*|branch)\s+(\.LBB\w+)\b")


def main_loops(asm: str, kernel_prefix: str) -> dict[str, tuple[int, int, int]]:
    """{instance symbol: (mfma, scratch, accvgpr)} of each kernel's main loop: of the innermost
    loops (a backward branch to a label, with no other loop inside), the one with the most MFMAs.
    (A persistent kernel's loop over tiles holds the main loop and so is not innermost.)"""
    lines = asm.split("\n")
    res = {}
    i = 0
    while i < len(lines):
        m = re.match(r"^(" + re.escape(kernel_prefix) + r"\w*):", lines[i])
        if not m:
            i += 1
            continue
        j = i
        while j < len(lines) and not lines[j].startswith(".Lfunc_end"):
            j += 1
        body = lines[i:j]
        where = {}
        for k, line in enumerate(body):
            lm = _LABEL.match(line)
            if lm:
                where[lm.group(1)] = k
        loops = []
        for e, line in enumerate(body):
            bm = _BRANCH.search(line)
            if bm and bm.group(1) in where and where[bm.group(1)] < e:
                loops.append((where[bm.group(1)], e))
        spans = {}
        for k, e in loops:  # one span per header: from the label to its last backward branch
            spans[k] = max(e, spans.get(k, e))
        inner = [(k, e) for k, e in spans.items()
                 if not any(k < k2 and e2 <= e for k2, e2 in spans.items() if (k2, e2) != (k, e))]
        best = (0, 0, 0)
        for k, e in inner:
            seg = body[k:e + 1]
            counts = (sum("v_mfma" in l for l in seg), sum("scratch_" in l for l in seg),
                      sum("v_accvgpr" in l for l in seg))
            best = max(best, counts)
        res[m.group(1)] = best
        i = j
    return res


def scan(source: str, kernel: str) -> dict[str, tuple[int, int, int]]:
    """Main-loop counts of every instance of `kernel` (unmangled name) in `source`."""
    return main_loops(device_asm(source), "_ZN4lora%d%s" % (len(kernel), kernel))


if __name__ == "__main__":
    for src, kern in (("fwd.hip", "fwd_mfma_kernel"), ("dx.hip", "dx_mfma_kernel")):
        for name, (mf, sc, av) in scan(src, kern).items():
            print(f"{name[:60]:60s} mfma {mf:4d}  scratch {sc:3d}  accvgpr {av:3d}")
    sys.exit(0)
