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

import hashlib
import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
LIB = PKG / "libw8a8.so"
SOURCES = ["w8a8_api.cpp", "rowwise.hip", "gemm.hip"]
# Headers the library's sources include (part of its build id).
HEADERS = [CSRC / "internal.h", CSRC / "rowwise.h", ROOT / "include" / "w8a8.h"]
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


def source_sha256(sources: list[str] | None = None) -> str:
    """SHA-256 over the named sources and the shared headers, in a fixed
    order: the build id compiled into the library (w8a8_build_id), compared
    by the binding against the files on disk to refuse a stale build."""
    h = hashlib.sha256()
    for f in [CSRC / s for s in (sources or SOURCES)] + HEADERS:
        h.update(f.name.encode() + b"\0" + f.read_bytes())
    return h.hexdigest()


def build(extra: list[str] | None = None, out: Path = LIB,
          verbose: bool = False, sources: list[str] | None = None) -> Path:
    """Compile every HIP source of the library into one shared object."""
    tmp = out.with_name(out.name + ".tmp")
    srcs = sources or SOURCES
    cmd = [HIPCC, *FLAGS, *(extra or []),
           f'-DW8A8_SOURCE_SHA256="{source_sha256(srcs)}"', "-o", str(tmp),
           *[str(CSRC / s) for s in srcs]]
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
