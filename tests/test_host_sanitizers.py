"""The C ABI's host code (argument validation, the plan, workspace carving,
the overlap checks) under AddressSanitizer and UndefinedBehaviorSanitizer, on
the CPU: a build of the library whose api.hip host code is instrumented
(device code unchanged) runs the whole ABI test module with the ASan runtime
preloaded; any sanitizer report aborts that process and fails this test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(lib):
    if not os.path.exists(lib):
        return True
    src = glob.glob(os.path.join(ROOT, "adamw_optimizer_step_amd", "csrc", "*")) + \
        [os.path.join(ROOT, "include", "muon_adamw.h")]
    return os.path.getmtime(lib) < max(os.path.getmtime(f) for f in src)


def test_abi_suite_under_host_asan_and_ubsan():
    from adamw_optimizer_step_amd import build as B
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    if _stale(B.SAN_LIB):
        B.build_host_sanitized(verbose=False)
    out = subprocess.run(["nm", "-D", B.SAN_LIB], capture_output=True, text=True).stdout
    assert "__asan_report" in out and "__ubsan_handle" in out, "the library is not instrumented"
    env = dict(os.environ, LD_PRELOAD=B.asan_runtime(), MA_LIBRARY=B.SAN_LIB,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout
