"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with both sanitizers on its host pass (device code is
unchanged) into a temporary folder, and the CPU tests of the ABI (symbol
exports, argument checks and status codes, workspace sizes) run against it
in a child process with the sanitizer runtime preloaded. A sanitizer report
aborts the child, and the test fails with its output.
"""
import os
import subprocess
import sys

import pytest

from w8a8_fp8_linear_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD_CHECK = """
import ctypes, os, sys
sys.path.insert(0, {root!r})
import w8a8_fp8_linear_amd as w8
assert w8.lib_path() == os.environ["W8A8_LIB"]
w8.lib()
maps = open("/proc/self/maps").read()
assert os.environ["W8A8_LIB"] in maps and "libclang_rt.asan" in maps
print("sanitized library loaded")
"""


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    try:
        runtime = b.sanitizer_runtime()
    except RuntimeError as e:  # pragma: no cover - toolchain without the runtime
        pytest.skip(str(e))
    lib = b.build(out=str(tmp_path / "libw8a8_sanitized.so"), sanitize_host=True)
    # the host code is instrumented: it calls into both sanitizers' runtimes
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    if nm.returncode == 0:
        assert "__asan_report_load8" in nm.stdout and "__ubsan_handle_" in nm.stdout
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["W8A8_LIB"] = lib
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["PYTHONDONTWRITEBYTECODE"] = "1"

    def run(args):
        return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                              timeout=600)

    res = run(["-c", CHILD_CHECK.format(root=ROOT)])
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    res = run(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
               os.path.join("tests", "test_abi_cpu.py")])
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert " passed" in res.stdout
