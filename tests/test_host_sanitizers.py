"""The library's host code (argument checks, workspace sizing, stack plans)
under AddressSanitizer and UndefinedBehaviorSanitizer, built with warnings as
errors, running the C-ABI tests of tests/test_abi.py and the random-plan
properties of tests/test_plan_properties.py in a child process with the ASan
runtime preloaded.  CPU only: no kernel is launched."""
import os
import subprocess
import sys

import pytest

from rank_gated_memory_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not installed")
def test_abi_tests_clean_under_host_sanitizers():
    lib = build.build_sanitized()
    env = dict(os.environ)
    env.update({
        "GSI_LIBRARY": lib,
        "LD_PRELOAD": build.asan_runtime(),
        # the interpreter itself is not instrumented: leak reports would be its own
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"),
                        os.path.join(ROOT, "tests", "test_plan_properties.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
