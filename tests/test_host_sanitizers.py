"""The host-only C-ABI tests (argument validation, planning, tune files, the owner planner)
once more against a build of the C++ front end with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only), in a subprocess with the sanitizer runtime
preloaded. Any report aborts that process, so the run must pass as the plain one does."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_and_planner_under_asan_ubsan():
    from matrix_orthogonalising_optimizer_muon_amd import build
    if not os.path.exists(build.HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    rt = build.asan_runtime()
    if rt is None:
        pytest.skip("no AddressSanitizer runtime in the ROCm toolchain")
    lib = build.build_asan()
    env = dict(os.environ, MUON_AMD_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_owner_plan.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "passed" in r.stdout and "failed" not in r.stdout
    # the library that ran was the instrumented one
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
