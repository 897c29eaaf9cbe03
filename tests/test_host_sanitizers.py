"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two child processes, each with its sanitizer runtime preloaded:
  - the C ABI's host tests (argument and layout checks, error codes, exports) against
    libvjsd built with the host pass of api.hip sanitized (clang; the kernels as usual);
  - the oracle's pins against the oracle's C source built with gcc's sanitizers.
Either suite failing, or any sanitizer report in its output, fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def run_suite(files, env_extra):
    env = dict(os.environ, OMP_NUM_THREADS="4", **env_extra)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           *[os.path.join(ROOT, "tests", f) for f in files]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in out, out[-2000:]
    for rep in REPORTS:
        assert rep not in out, out[-4000:]


def test_abi_host_checks_under_asan_ubsan():
    import importlib.util

    spec = importlib.util.spec_from_file_location(
        "_vjsd_build", os.path.join(ROOT, "vocab_sharded_softmax_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    try:
        lib, rt = b.build_host_sanitized(), b.asan_runtime()
    except RuntimeError as e:  # no HIP toolchain on this host
        pytest.skip(str(e))
    run_suite(["test_abi_host.py", "test_binding_host.py"],
              {"LD_PRELOAD": rt, "VJSD_LIB": lib,
               "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
               "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})


def test_oracle_pins_under_asan_ubsan(tmp_path):
    import oracle

    lib = oracle.build_sanitized(str(tmp_path))
    rt = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                        text=True, check=True).stdout.strip()
    run_suite(["test_oracle_pins.py", "test_oracle_loss_pins.py", "test_oracle_topk_pins.py",
               "test_oracle_ce_pins.py", "test_oracle_linear_pins.py"],
              {"LD_PRELOAD": rt, "VJSD_ORACLE_LIB": lib,
               "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
               "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
