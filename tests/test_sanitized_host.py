"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two legs, each in a child process that preloads the matching ASan runtime:

* the oracle (oracle.c, gcc -fsanitize=address,undefined) runs every pin
  of tests/test_oracle_pins.py;
* a host-only build of the library's sources (hipcc, the sanitizers on the
  host pass; no device code, nothing is launched) runs every C-ABI
  validation case of tests/test_abi.py.

Any out-of-bounds access, use after free or undefined behaviour aborts the
child, and the test fails with its report.  Leak checking is off: the
Python interpreter itself keeps memory until exit.
"""
import os
import subprocess
import sys

import pytest

import oracle
from transformer_scaled_dot_fwd_amd import build as hip_build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _run_child(env_extra, test_file):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                           "-p", "no:cacheprovider", os.path.join(HERE, test_file)],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = proc.stdout[-4000:] + proc.stderr[-4000:]
    assert proc.returncode == 0, out
    assert "passed" in proc.stdout, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = oracle.build_checked(str(tmp_path / "liboracle_checked.so"))
    _run_child({"LD_PRELOAD": oracle.checked_runtime(), "ORACLE_CHECKED_LIBRARY": lib},
               "test_oracle_pins.py")


def test_c_abi_validation_under_sanitizers(tmp_path):
    try:
        runtime = hip_build.asan_runtime()
    except (RuntimeError, subprocess.CalledProcessError, FileNotFoundError) as e:
        pytest.fail(f"the compiler's ASan runtime is missing: {e}")
    lib = hip_build.build_host_checked(str(tmp_path))
    _run_child({"LD_PRELOAD": runtime, "MHA_HOST_CHECKED_LIBRARY": lib}, "test_abi.py")
