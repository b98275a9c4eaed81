"""Build the CPU oracle shared object with gcc.

Test infrastructure: the product library never uses what this builds.
Flags keep every binary32 operation a single IEEE rounding (no FMA
contraction, no fast-math) and avoid -march=native so the object runs on
any x86-64 host it is copied to.
"""
from __future__ import annotations

import os
import subprocess
from pathlib import Path

HERE = Path(__file__).resolve().parent
SRC = HERE / "w8a8_oracle.c"
LIB = HERE / "libw8a8_oracle.so"

CFLAGS = [
    "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
    "-Wall", "-Wextra",
]


def extra_cflags() -> list[str]:
    """Flags added to every oracle build from W8A8_ORACLE_CFLAGS (the
    sanitizer test builds its copies with -fsanitize=undefined)."""
    return os.environ.get("W8A8_ORACLE_CFLAGS", "").split()


def build_from(src: Path, out: Path) -> Path:
    """Compile one oracle source file into a shared object."""
    tmp = out.with_suffix(".so.tmp")
    cmd = ["gcc", *CFLAGS, *extra_cflags(), "-I", str(HERE), "-o", str(tmp),
           str(src), "-lm"]
    subprocess.run(cmd, check=True)
    tmp.replace(out)
    return out


def build() -> Path:
    """Compile oracle/w8a8_oracle.c into oracle/libw8a8_oracle.so."""
    return build_from(SRC, LIB)


if __name__ == "__main__":
    print(build())
