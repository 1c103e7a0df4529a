"""Host-sanitized variant of the library, for checking the C ABI's host code on the CPU.

lora_api.cpp (argument validation, workspace layout, dispatch) is compiled with AddressSanitizer
and UndefinedBehaviorSanitizer on its host code only (the device code of every kernel is left as
it is) and linked with the kernel objects of the regular build into
qlora_fine_tuning_amd/liblora_mi355x_hostsan.so.  The library expects the sanitizer runtime to be
loaded first (LD_PRELOAD of runtime_path()); lora.load() picks it up when QLORA_AMD_LIB names it.
Usage:

    python -m qlora_fine_tuning_amd.build_sanitized
"""
from __future__ import annotations

import glob
import os
import sys

from qlora_fine_tuning_amd import build as _b

LIB_PATH = os.path.join(_b.PKG, "liblora_mi355x_hostsan.so")
SAN_DIR = os.path.join(_b.BUILD_DIR, "hostsan")
API = os.path.join(_b.CSRC, "lora_api.cpp")
CLANG = "/opt/rocm/llvm/bin/clang++"
ROCM_LIB = "/opt/rocm/lib"


def runtime_path() -> str:
    """The shared AddressSanitizer runtime (with the UndefinedBehaviorSanitizer handlers)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("the clang AddressSanitizer runtime is not installed")
    return hits[-1]


def build(jobs: int = 8, verbose: bool = False) -> str:
    """Compile lora_api.cpp with host-only sanitizers and link it with the kernel objects (built
    first if missing); returns the library's path."""
    objs = [os.path.join(_b.BUILD_DIR, os.path.basename(s) + ".o") for s in _b.sources() if s != API]
    if not all(os.path.exists(o) for o in objs):
        _b.build(jobs, verbose)
    os.makedirs(SAN_DIR, exist_ok=True)
    api_obj = os.path.join(SAN_DIR, "lora_api.cpp.o")
    # every sanitizer flag goes to the host compilation only
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f if f != "-O3" else "-O1" for f in _b.HIP_FLAGS]
    _b._run([_b._hipcc(), *flags, *san, "-g", "-x", "hip", "-c", API, "-o", api_obj], verbose)
    tmp = LIB_PATH + ".tmp"
    link_san = ["-fsanitize=address,undefined", "-shared-libsan"]
    _b._run([CLANG, "-shared", "-fPIC", *link_san, "-o", tmp, api_obj, *objs, "-L", ROCM_LIB, "-lamdhip64",
             f"-Wl,-rpath,{ROCM_LIB}"], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    sys.exit(0)
