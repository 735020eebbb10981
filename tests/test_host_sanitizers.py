"""The oracle and the C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

CPU only.  The oracle is rebuilt with gcc's sanitizers and its pin tests run against it; the
library's host code (argument validation, workspace layout, launch set-up) is rebuilt with
clang's (no device code) and the C-ABI host tests run against it.  Each in a child process
that preloads the matching sanitizer runtime; any report fails the child and so the test.
"""
import os
import subprocess
import sys

import pytest

import oracle
from bit_moe_expert_route_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_pytest(test_file, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m",
           "not gpu", os.path.join(ROOT, "tests", test_file)]
    r = subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def _instrumented(lib):
    """The library calls into the sanitizer runtimes (so it cannot even load without them)."""
    r = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "__asan_" in r.stdout and "__ubsan_" in r.stdout


def _gcc_asan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path):
        pytest.skip("gcc's libasan not found")
    return path


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = oracle.build(out=str(tmp_path / "libmoe_oracle_san.so"), sanitize=True)
    _instrumented(lib)
    out = _run_pytest("test_oracle_pins.py",
                      {"LD_PRELOAD": _gcc_asan(), "MOE_ORACLE_LIB": lib})
    assert "passed" in out


def test_capi_host_checks_under_asan_ubsan(tmp_path):
    try:
        rt = libbuild.sanitizer_runtime()
    except RuntimeError as exc:
        pytest.skip(str(exc))
    lib = libbuild.build(out=str(tmp_path / "libmoe_mx_san.so"), sanitize_host=True)
    _instrumented(lib)
    out = _run_pytest("test_capi_host.py", {"LD_PRELOAD": rt, "MOE_LIB_PATH": lib})
    assert "passed" in out
