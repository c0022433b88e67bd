"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt with its host code instrumented (libmoe_ffn_san.so,
built here when missing or older than the sources), and the tests of
test_abi_cpu.py (exports, every argument rule, the last-error text) run
against it in a child process that preloads the ASan runtime and loads that
build through MOE_FFN_LIB.  Any sanitizer report ends the child with a
non-zero status, which fails this test.  No call reaches a kernel launch.
"""
import os
import subprocess
import sys

import pytest

from expert_ffn_dispatch_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san_env():
    rt = B.asan_runtime()
    if not rt:
        pytest.skip("the compiler's shared ASan runtime is not installed")
    if not B.sanitized_is_current():
        B.build_sanitized()
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = rt + (":" + pre if pre else "")   # the runtime must come first
    env["MOE_FFN_LIB"] = B.SAN_LIB
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    return env


def _run(env, args):
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


def test_sanitizers_are_live(san_env):
    """The child resolves the ASan entry point, loads the instrumented build,
    and that build references the sanitizer runtime."""
    code = ("import ctypes\n"
            "from expert_ffn_dispatch_amd import _lib\n"
            "ctypes.CDLL(None)['__asan_init']\n"
            "lib = _lib.load()\n"
            "assert _lib.LIB_PATH.endswith('libmoe_ffn_san.so'), _lib.LIB_PATH\n"
            "assert lib.moe_abi_version() == 1\n"
            "print('ok')\n")
    r = _run(san_env, ["-c", code])
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
    syms = subprocess.run(["nm", "-D", B.SAN_LIB], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms


def test_abi_rules_under_sanitizers(san_env):
    r = _run(san_env, ["-m", "pytest", "tests/test_abi_cpu.py", "-q", "-p", "no:cacheprovider"])
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
