"""Build libw8a8.so (the C-ABI library) for gfx950 with hipcc, in-tree.

The shared object lands next to this file, where the Python binding loads
it.  hipcc cross-compiles without a GPU.  Flags:
  * --offload-arch=gfx950 only (no other target, no host fallback);
  * -ffp-contract=off: the epilogue's binary32 operations are rounded one by
    one, never fused into FMAs;
  * -Xclang -target-feature -Xclang -packed-fp32-ops: no packed FP32 VALU
    instructions are generated (the host pass warns that it does not know
    the feature, which is harmless);
  * no fast-math: FP32 division stays correctly rounded and subnormals are
    kept.
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libw8a8.so"
SOURCES = ["w8a8_api.cpp", "rowwise.hip", "gemm.hip"]
# Measurement support, not part of the library: the register-only MFMA
# rate on given code matrices (loaded by bench.py only).
CEILING_LIB = PKG / "libw8a8_ceiling.so"
CEILING_SOURCES = ["mfma_ceiling.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
    "-packed-fp32-ops", "-Wall", "-Wno-unused-function",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]


def build(extra: list[str] | None = None, out: Path = LIB,
          verbose: bool = False, sources: list[str] | None = None) -> Path:
    """Compile every HIP source of the library into one shared object."""
    tmp = out.with_name(out.name + ".tmp")
    cmd = [HIPCC, *FLAGS, *(extra or []), "-o", str(tmp),
           *[str(CSRC / s) for s in (sources or SOURCES)]]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)
    tmp.replace(out)
    return out


def build_ceiling(verbose: bool = False) -> Path:
    """Compile the MFMA-ceiling measurement kernel (libw8a8_ceiling.so)."""
    return build(out=CEILING_LIB, verbose=verbose, sources=CEILING_SOURCES)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_ceiling(verbose=True))
