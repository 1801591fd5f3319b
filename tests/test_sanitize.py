"""The host-side code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

Two runs, each in a child process because each needs its sanitizer runtime preloaded:
  * the oracle, built by gcc with -fsanitize=address,undefined (LA_ORACLE_SANITIZE=1), under its
    own pin tests (test_oracle_pins.py, test_oracle_bwd_pins.py);
  * the library's host code (argument validation, planning arithmetic, error paths), built by
    hipcc with the sanitizers on the host side only (chunked_scan_amd.build.build_sanitized), under
    the C-ABI tests (test_abi.py, test_abi_fuzz.py).
Any sanitizer report ends the child with a non-zero status (UBSan reports are made fatal).  The
same commands, run by hand:
  LA_ORACLE_SANITIZE=1 LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \\
      python -m pytest tests/test_oracle_pins.py tests/test_oracle_bwd_pins.py
  python -c "from chunked_scan_amd import build; build.build_sanitized()"
  LACHUNK_LIB=_build/san/liblachunk.so LD_PRELOAD=$(hipcc --print-file-name=libclang_rt.asan-x86_64.so) \\
      ASAN_OPTIONS=detect_leaks=0 python -m pytest tests/test_abi.py tests/test_abi_fuzz.py
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                                reason="the C-ABI fuzz uses fake device addresses: runs only without a GPU")


def _run(env_extra, tests, timeout=900):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *tests]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]


def test_oracle_under_sanitizers():
    if not shutil.which("gcc"):
        pytest.skip("gcc is not installed")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc's libasan is not installed")
    _run({"LA_ORACLE_SANITIZE": "1", "LD_PRELOAD": asan},
         ["tests/test_oracle_pins.py", "tests/test_oracle_bwd_pins.py"])


def test_library_host_code_under_sanitizers():
    from chunked_scan_amd import build

    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc is not installed")
    lib = build.build_sanitized(verbose=False)
    _run({"LACHUNK_LIB": lib, "LD_PRELOAD": build.asan_runtime()},
         ["tests/test_abi.py", "tests/test_abi_fuzz.py"])
