"""The oracle's pin tests once more against oracle.c built with AddressSanitizer and
UndefinedBehaviorSanitizer (every report fatal), in a child process that loads the ASan
runtime first. Host code only; skipped where gcc has no sanitizer runtimes."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_asan.so"))
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=f"{asan} {ubsan}", OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", f) for f in
             ("test_oracle_formats.py", "test_oracle_quant.py", "test_oracle_layer.py", "test_oracle_fp8.py")]
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-3000:]
    assert "passed" in p.stdout
