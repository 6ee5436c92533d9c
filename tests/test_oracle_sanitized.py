"""The CPU oracle's pins run again with the oracle built under AddressSanitizer
and UndefinedBehaviorSanitizer (gcc, host code only): an out-of-bounds access,
a use of freed memory, a signed overflow, a misaligned or out-of-range shift
anywhere in moe_oracle.c aborts the run."""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_replica_pins.py", "tests/test_oracle_mxfp8_pins.py"]


def test_oracle_pins_under_asan_and_ubsan():
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not libasan or not Path(libasan).exists():
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    env = dict(os.environ, MOE_ORACLE_SANITIZE="1", LD_PRELOAD=libasan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    build = subprocess.run([sys.executable, "-c", "import oracle; oracle.build(force=True)"], cwd=ROOT, env=env,
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([sys.executable, "-m", "pytest", *PINS, "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert run.returncode == 0, (run.stdout[-3000:], run.stderr[-3000:])
    assert "passed" in run.stdout
