"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A variant of the library with the host code instrumented (device code is
compiled as usual) is built when missing or older than the sources, then
tests/test_abi_cpu.py (argument validation, workspace sizes, error paths,
every exported symbol) runs against it in a child process with the ASan
runtime preloaded. Any sanitizer report fails the run (UBSan does not
recover). No GPU is involved."""

import os
import subprocess
import sys

import pytest

from precision_rl_nvfp4_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale():
    if not os.path.exists(B.SAN_LIB):
        return True
    t = os.path.getmtime(B.SAN_LIB)
    srcs = B.SOURCES + [os.path.join(B.CSRC, "trace_fp4_internal.h"), os.path.join(ROOT, "include", "trace_fp4.h")]
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.fixture(scope="module")
def san_lib():
    try:
        B.hipcc()
        rt = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    if _stale():
        B.build_sanitized()
    return B.SAN_LIB, rt


def test_sanitized_build_is_instrumented(san_lib):
    lib, _ = san_lib
    out = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_" in out and "__ubsan_handle_" in out


def test_abi_cpu_tests_pass_under_host_sanitizers(san_lib):
    lib, rt = san_lib
    code = ("import sys\n"
            f"sys.path.insert(0, {ROOT!r})\n"
            "from precision_rl_nvfp4_amd import _abi\n"
            f"_abi.LIB_PATH = {lib!r}\n"
            "import pytest\n"
            f"sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', {os.path.join(ROOT, 'tests', 'test_abi_cpu.py')!r}]))\n")
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
