"""The C-ABI tests run against a build whose host dispatch (fa_api.hip:
argument checks, overlap tests, planners, the workspace and scratch maps) is
compiled with AddressSanitizer and UndefinedBehaviorSanitizer.  Any report
aborts the child interpreter and fails this test."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "exact_io_aware_02_amd")


def _build_module():
    sys.path.insert(0, PKG)
    try:
        import build
    finally:
        sys.path.remove(PKG)
    return build


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_abi_suite_under_asan_and_ubsan():
    build = _build_module()
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("the compiler's shared ASan runtime is not installed")
    lib = build.build_host_sanitized()
    nm = shutil.which("nm") or shutil.which("llvm-nm")
    if nm:
        syms = subprocess.run([nm, "-D", lib], stdout=subprocess.PIPE, text=True).stdout
        assert "__asan_report_load" in syms and "__ubsan_handle" in syms, "the build is not instrumented"
    preload = " ".join(x for x in (rt, os.environ.get("LD_PRELOAD", "")) if x)
    env = dict(os.environ, FA_LIBRARY=lib, LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys, pytest, exact_io_aware_02_amd as fa; "
            f"assert fa.LIB_PATH == {lib!r}, fa.LIB_PATH; "
            "sys.exit(pytest.main(['tests/test_abi.py', '-q', '-x', '-p', 'no:cacheprovider']))")
    p = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=600)
    assert p.returncode == 0, p.stdout[-4000:]
    assert " passed" in p.stdout and "ERROR: AddressSanitizer" not in p.stdout
