"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

Two builds of ``oracle/oracle.c``, both with every sanitizer error fatal:
- ``tests/oracle_sanitize_driver.c`` linked with the oracle under ASan + UBSan (static runtimes), which
  drives every entry point at its edge shapes with exactly sized heap buffers;
- the oracle as a shared library under UBSan, loaded through ``RL_ORACLE_LIB`` by the oracle's pin files
  in a fresh interpreter, so that every pin case runs on the sanitized code. (ASan cannot be loaded into
  an uninstrumented interpreter without preloading its runtime, hence the driver for memory errors.)
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-static-libasan", "-static-libubsan"]


def test_driver_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-Wall", "-Wextra", *SAN, "-o", exe,
                           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"), "-lm"])
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0"))
    assert res.returncode == 0 and "sanitize ok" in res.stdout, res.stderr[-3000:]


def test_pin_cases_under_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_ubsan.so")
    flags = [f for f in oracle.GCC_FLAGS if not f.startswith("-O")]
    subprocess.check_call(["gcc", "-O1", "-g", *flags, "-fsanitize=undefined", "-fno-sanitize-recover=all", "-o",
                           lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    pins = sorted(p for p in glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))
                  if not p.endswith(("_mutants.py", "_sanitize.py")))
    env = dict(os.environ, RL_ORACLE_LIB=lib, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               PYTHONDONTWRITEBYTECODE="1")
    res = subprocess.run([sys.executable, "-m", "pytest", *pins, "-q", "-m", "not gpu"], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=1200)
    assert res.returncode == 0, (res.stdout[-2000:], res.stderr[-3000:])
