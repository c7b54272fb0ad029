"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds _build/asan/libmoe.so (moe_abi.hip's host code instrumented, host
passes only; device code as usual) and runs the ABI tests of test_abi.py
against it in a child process that preloads the clang sanitizer runtime:
argument validation, workspace sizing and the status/error strings, with any
out-of-bounds access, use after free or undefined behaviour aborting the run.
No GPU is involved (those tests stop before any device call).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    from mixture_experts_layer_28_amd import build as B
    try:
        runtime = B.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = B.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=runtime, MOE_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return lib, env


def test_sanitized_build_is_instrumented_and_runtime_active(sanitized):
    lib, env = sanitized
    code = ("import ctypes, mixture_experts_layer_28_amd as moe; L = moe.lib(); "
            "rt = ctypes.CDLL(None); rt.__asan_region_is_poisoned; "
            "print('abi', L.moe_abi_version())")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "abi" in r.stdout
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True)
    assert "__asan_report" in nm.stdout and "__ubsan_handle" in nm.stdout


def test_abi_tests_pass_under_sanitizers(sanitized):
    _, env = sanitized
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi.py", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
