"""Build the gfx950 HIP library in-tree: qlora_fine_tuning_amd/liblora_mi355x.so.

Every source under csrc/ is compiled by hipcc for gfx950 only and linked into one shared
library that exports the C ABI declared in include/lora.h.  Usage:

    python -m qlora_fine_tuning_amd.build [-j JOBS] [-v]
"""
from __future__ import annotations

import argparse
import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "liblora_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

# Packed fp32 VALU ops are disabled (the compiler would otherwise form them from scalar or
# float2 code); fp32 division and sqrt are correctly rounded, which the int4 quantiser's
# exact code decisions rely on.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-munsafe-fp-atomics",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source extra flags.  The MFMA kernels keep their main accumulators in AGPRs through
# inline asm; the builtin MFMAs of their small rank-R panels are put in VGPRs so that the two
# never compete for the AGPR file.
EXTRA_FLAGS = {
    "fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "dx.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return out


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "lora_api.cpp")]


def build(jobs: int = 8, verbose: bool = False) -> str:
    """Compile every source and link the library; returns its path.  Always rebuilds."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        extra = EXTRA_FLAGS.get(os.path.basename(src), [])
        cmd = [hipcc, *HIP_FLAGS, *extra, "-x", "hip", "-c", src, "-o", obj]
        _run(cmd, verbose)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("-j", "--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))


if __name__ == "__main__":
    sys.exit(main())
