"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU:
lora_api.cpp (validation, workspace layouts, dispatch) is built with host-only sanitizers
(qlora_fine_tuning_amd.build_sanitized) and test_abi.py runs against that library in a child
process with the sanitizer runtime preloaded.  Any sanitizer report, or any failing check, fails
this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_sanitizers(tmp_path):
    from qlora_fine_tuning_amd import build_sanitized as bs

    try:
        runtime = bs.runtime_path()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = bs.build()
    preload = runtime + (":" + os.environ["LD_PRELOAD"] if os.environ.get("LD_PRELOAD") else "")
    env = dict(os.environ, LD_PRELOAD=preload, QLORA_AMD_LIB=lib,
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={tmp_path}/asan",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={tmp_path}/ubsan")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = sorted(p for p in tmp_path.iterdir() if p.name.startswith(("asan", "ubsan")))
    text = "".join(p.read_text() for p in reports)
    assert r.returncode == 0 and not reports, (r.stdout[-3000:] + r.stderr[-3000:] + text[:4000])
    assert " passed" in r.stdout
