"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

* The C ABI's argument checks (csrc/validate.cpp, the same object the
  library links) are built with both sanitizers together with
  tests/sanitize/validators_check.cpp, which drives them through the ABI
  tests' rejection and acceptance cases plus extreme sizes and strides (no
  size product may overflow).
* The oracle (oracle/mxoracle.c) is built with both sanitizers and the
  oracle test files run against it in a child process with the ASan
  runtime preloaded.
Either passes only with no sanitizer report (UB aborts the run)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp8_block_scaled_gemm_amd", "csrc")
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="no host C/C++ compiler")


def _asan_runtime() -> str:
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not path or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("no ASan runtime for gcc")
    return path


def test_argument_checks_under_sanitizers(tmp_path):
    exe = tmp_path / "validators_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(CSRC, "validate.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "validators_check.cpp"),
                    "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out
    assert not any(r in out for r in REPORTS), out
    assert "0 mismatches" in out


@pytest.mark.slow
def test_oracle_suite_under_sanitizers():
    env = dict(os.environ)
    env.update(LD_PRELOAD=_asan_runtime(), MXG_ORACLE_SANITIZE="1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", PYTHONDONTWRITEBYTECODE="1")
    tests = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith("test_oracle_") and f.endswith(".py"))
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert not any(r in out for r in REPORTS), out[-4000:]
    assert " passed" in out
