"""The CPU oracle under sanitizers.

* AddressSanitizer + UndefinedBehaviorSanitizer: a C driver
  (tests/oracle_sanitize_driver.c) calls every oracle entry point on
  exactly sized heap buffers -- ragged shapes, zero rows, subnormals,
  every error path -- in an executable built with both sanitizers; any
  report aborts it.
* UndefinedBehaviorSanitizer under the Python suites: the oracle is
  rebuilt as a shared object with -fsanitize=undefined (no preloaded
  runtime needed) and the pin suite and the mutant suite run against that
  build in a child pytest (the mutants are built with the same flags).
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
ORACLE = ROOT / "oracle"
SAN_ABORT = ["-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def test_oracle_entry_points_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-frounding-math",
           "-fsanitize=address,undefined", *SAN_ABORT,
           "-I", str(ORACLE), "-o", str(exe),
           str(ORACLE / "w8a8_oracle.c"),
           str(ROOT / "tests" / "oracle_sanitize_driver.c"), "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, OMP_NUM_THREADS="3",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env,
                         timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "oracle sanitizer driver: ok" in res.stdout
    assert "runtime error" not in res.stderr


def test_pins_and_mutants_under_ubsan(tmp_path):
    flags = "-fsanitize=undefined " + " ".join(SAN_ABORT)
    lib = tmp_path / "liboracle_ubsan.so"
    env = dict(os.environ, W8A8_ORACLE_CFLAGS=flags)
    subprocess.run([sys.executable, "-c",
                    "import sys; from pathlib import Path; "
                    "from oracle import build as b; "
                    "b.build_from(b.SRC, Path(sys.argv[1]))", str(lib)],
                   check=True, cwd=ROOT, env=env)
    env.update(W8A8_ORACLE_LIB=str(lib),
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
         "tests/test_oracle_pins.py", "tests/test_oracle_mutants.py"],
        capture_output=True, text=True, cwd=ROOT, env=env, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "runtime error" not in out, out[-4000:]
    assert " passed" in out
