"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
the CPU ABI tests (argument validation of every entry point, planning, the
binding's checks) run against liblutq_san.so, a build of the library whose
host code is instrumented (device code as in liblutq.so), with the clang
ASan runtime preloaded. Any sanitizer report fails the run."""

import os
import subprocess
import sys

import pytest

from weight_only_lut_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_clean_under_host_sanitizers():
    runtime = build.asan_runtime()
    if runtime is None:
        pytest.skip("clang ASan runtime not found")
    if not os.path.exists(build.SAN_LIB):
        pytest.skip("liblutq_san.so not built (python -m weight_only_lut_amd.build)")
    nm = subprocess.run(["nm", "-D", build.SAN_LIB], capture_output=True, text=True).stdout
    assert "__asan_report_load" in nm and "__ubsan_handle_" in nm, "host code is not instrumented"
    env = dict(os.environ)
    env.update({"LUTQ_LIBRARY": build.SAN_LIB, "LD_PRELOAD": runtime,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-3000:]
    assert " passed" in out
