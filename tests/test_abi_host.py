"""The C-ABI library on the host: it loads, exports every symbol that
include/w8a8.h declares, and rejects bad arguments before launching
anything.  No kernel is launched here: every call below fails validation,
which happens before the library touches the device.  Pointers are fake
addresses that are never dereferenced."""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

import pytest

from w8a8_int8_gemm_amd import binding as B

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "w8a8.h"

OK, NULL, SHAPE, ALIGN, WORKSPACE, OUT_DTYPE, ALIAS, DEVICE, HIP = range(9)

# Fake, well-separated, 4 KiB-aligned device addresses.
A = 0x10_0000_0000
BUF = {name: A + i * 0x1_0000_0000 for i, name in enumerate(
    ["x", "aq", "sa", "w", "sw", "bias", "out", "ws"])}


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a8_\w+)\s*\(", text)))


def test_header_declares_expected_api():
    names = declared_functions()
    for n in ["w8a8_quantize_act", "w8a8_gemm", "w8a8_linear",
              "w8a8_workspace_bytes", "w8a8_status_string"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(B.LIB_PATH))
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"
    # and the binding wraps exactly the declared set
    assert sorted(B.SIGNATURES) == declared_functions()


def test_status_strings():
    lib = B.lib()
    seen = set()
    for code in range(9):
        s = lib.w8a8_status_string(code)
        assert s and s not in seen
        seen.add(s)
    assert lib.w8a8_status_string(99) == b"unknown status"


def gemm(**kw):
    a = dict(aq=BUF["aq"], sa=BUF["sa"], w=BUF["w"], sw=BUF["sw"],
             bias=BUF["bias"], out=BUF["out"], dt=0, M=64, N=256, K=256,
             ws=BUF["ws"], wsb=1 << 30)
    a.update(kw)
    return B.lib().w8a8_gemm(a["aq"], a["sa"], a["w"], a["sw"], a["bias"],
                             a["out"], a["dt"], a["M"], a["N"], a["K"],
                             a["ws"], a["wsb"], None)


def quant(**kw):
    a = dict(x=BUF["x"], M=4, K=5376, q=BUF["aq"], s=BUF["sa"])
    a.update(kw)
    return B.lib().w8a8_quantize_act(a["x"], a["M"], a["K"], a["q"], a["s"],
                                     None)


def linear(**kw):
    a = dict(x=BUF["x"], w=BUF["w"], sw=BUF["sw"], bias=BUF["bias"],
             y=BUF["out"], M=64, N=256, K=256, ws=BUF["ws"], wsb=1 << 30)
    a.update(kw)
    return B.lib().w8a8_linear(a["x"], a["w"], a["sw"], a["bias"], a["y"],
                               a["M"], a["N"], a["K"], a["ws"], a["wsb"],
                               None)


@pytest.mark.parametrize("kw,code", [
    (dict(aq=None), NULL), (dict(sa=None), NULL), (dict(w=None), NULL),
    (dict(sw=None), NULL), (dict(out=None), NULL),
    (dict(M=0), SHAPE), (dict(M=-5), SHAPE), (dict(N=0), SHAPE),
    (dict(N=100), SHAPE), (dict(N=5376 + 64), SHAPE), (dict(K=5376 + 8), SHAPE),
    (dict(K=0), SHAPE), (dict(K=B.MAX_K + 128), SHAPE), (dict(M=1 << 31), SHAPE),
    # tile grid beyond 2^32 work-items: 8388608 x 84 tiles of 512
    (dict(M=(1 << 31) - 1, N=21504, wsb=1 << 62), SHAPE),
    (dict(dt=3), OUT_DTYPE), (dict(dt=-1), OUT_DTYPE),
    (dict(aq=BUF["aq"] + 8), ALIGN), (dict(w=BUF["w"] + 4), ALIGN),
    (dict(out=BUF["out"] + 2), ALIGN), (dict(sw=BUF["sw"] + 2), ALIGN),
    (dict(sa=BUF["sa"] + 2), ALIGN), (dict(bias=BUF["bias"] + 1), ALIGN),
    (dict(out=BUF["aq"]), ALIAS), (dict(out=BUF["w"] + 1024), ALIAS),
    (dict(out=BUF["sw"] - 16), ALIAS), (dict(out=BUF["bias"]), ALIAS),
])
def test_gemm_rejects(kw, code):
    assert gemm(**kw) == code


def test_gemm_workspace_checks():
    # M = 128 plans split-K over 64 x 128 tiles and needs a workspace
    need = B.gemm_workspace_bytes(128, 5376, 5376)
    assert need > 0
    assert gemm(M=128, N=5376, K=5376, ws=None, wsb=0) == WORKSPACE
    assert gemm(M=128, N=5376, K=5376, wsb=need - 1) == WORKSPACE
    assert gemm(M=128, N=5376, K=5376, ws=BUF["ws"] + 8, wsb=need) == ALIGN
    assert gemm(M=128, N=5376, K=5376, ws=BUF["out"], wsb=need) == ALIAS


def test_gemm_accepts_planned_alignments():
    """Scales need only 4-byte alignment, the bias 2-byte and the workspace
    16-byte (a channel slice of larger arrays): such calls pass validation
    and reach the device check (no device here)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    assert gemm(sw=BUF["sw"] + 4, bias=BUF["bias"] + 2) == DEVICE
    assert gemm(M=128, N=5376, K=5376, ws=BUF["ws"] + 16,
                wsb=B.gemm_workspace_bytes(128, 5376, 5376)) == DEVICE
    assert linear(sw=BUF["sw"] + 12, bias=BUF["bias"] + 6,
                  ws=BUF["ws"] + 16) == DEVICE
    # K up to the INT32 bound through linear (the quantizer takes it too)
    assert linear(M=3, N=256, K=B.MAX_K) == DEVICE
    assert quant(K=B.MAX_K) == DEVICE


def test_workspace_sizes():
    # 256x256 tiles: a full number of 256-tile waves needs no workspace; a
    # short last wave (t tiles) is split s = min(256 // t, K // 512) ways
    # into INT32 tiles of its own when s >= 2 (each slice at least 512
    # bytes of K, four 128-byte stages).
    tile = 256 * 256 * 4
    g = B.gemm_workspace_bytes
    assert g(4096, 4096, 5376) == 0           # 256 tiles
    assert g(19077, 21504, 5376) == 0         # 6300: s = 1
    assert g(19077, 5376, 5376) == 6 * 39 * tile   # 1575
    assert g(37503, 5376, 21504) == 17 * 15 * tile  # 3087
    assert g(4097, 4096, 1664) == 3 * 16 * tile    # 13 stages
    assert g(4097, 4096, 1024) == 2 * 16 * tile
    assert g(4097, 4096, 512) == 0            # 4 stages
    # at most 64 tokens: one launch of the single-launch kernel, no partial
    # sums; 65 to a few hundred tokens: 64 x 128 tiles split over K
    for M in (1, 17, 32, 33, 64):
        for N in (128, 5376, 16384):
            assert g(M, N, 5376) == 0
    assert g(64, 21504, 5376) == 0          # 168 tiles of 64 x 128, unsplit
    assert g(64, 5376, 21504) > 0           # long K: split-K tiles
    ws = g(128, 5376, 5376)
    assert ws % (128 * 5376 * 4) == 0 and ws // (128 * 5376 * 4) >= 2
    assert g(64, 100, 5376) == 0  # rejected shape
    # w8a8_workspace_bytes: the codes and scales linear stages, each at a
    # 256-byte offset, plus the GEMM's partial sums (so it serves both)
    r = lambda v: (v + 255) // 256 * 256
    for M, N, K in [(19077, 5376, 5376), (64, 5376, 5376), (300, 384, 640),
                    (3, 256, B.MAX_K)]:
        assert B.workspace_bytes(M, N, K) == r(M * K) + r(4 * M) + g(M, N, K)
    assert B.workspace_bytes(64, 100, 5376) == 0
    assert B.workspace_bytes(1 << 24, 128, 128) == 0  # beyond the quantizer


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(q=None), NULL), (dict(s=None), NULL),
    (dict(M=0), SHAPE), (dict(M=1 << 24), SHAPE),
    (dict(K=4), SHAPE), (dict(K=5377), SHAPE),
    (dict(K=B.MAX_K + 8), SHAPE),
    (dict(x=BUF["x"] + 8), ALIGN), (dict(q=BUF["aq"] + 4), ALIGN),
    (dict(s=BUF["sa"] + 1), ALIGN),
    (dict(q=BUF["x"] + 16), ALIAS), (dict(s=BUF["aq"] + 64), ALIAS),
])
def test_quantize_rejects(kw, code):
    assert quant(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(y=None), NULL), (dict(M=0), SHAPE),
    (dict(K=B.MAX_K + 128), SHAPE), (dict(ws=None), WORKSPACE),
    (dict(wsb=100), WORKSPACE), (dict(ws=BUF["ws"] + 8), ALIGN),
    (dict(sw=BUF["sw"] + 2), ALIGN), (dict(bias=BUF["bias"] + 1), ALIGN),
    (dict(x=BUF["x"] + 2), ALIGN), (dict(y=BUF["x"]), ALIAS),
    (dict(ws=BUF["w"]), ALIAS),
])
def test_linear_rejects(kw, code):
    assert linear(**kw) == code


def test_glue_rejects():
    lib = B.lib()
    assert lib.w8a8_silu_bf16(None, BUF["out"], 8, None) == NULL
    assert lib.w8a8_silu_bf16(BUF["x"], BUF["out"], 9, None) == SHAPE
    assert lib.w8a8_silu_bf16(BUF["x"] + 2, BUF["out"], 8, None) == ALIGN
    assert lib.w8a8_silu_bf16(BUF["x"], BUF["x"] + 16, 64, None) == ALIAS
    assert lib.w8a8_pow2_renorm(BUF["x"], BUF["out"], 0, 8, None) == SHAPE
    assert lib.w8a8_pow2_renorm(BUF["x"], BUF["x"] + 16, 4, 64, None) == ALIAS
    assert lib.w8a8_quantize_act_silu(BUF["x"], 4, 12, BUF["aq"], BUF["sa"],
                                      None) == SHAPE
    assert lib.w8a8_quantize_act_silu(BUF["x"], 4, B.GLUE_MAX_K + 8,
                                      BUF["aq"], BUF["sa"], None) == SHAPE


def test_weight_and_gated_glue_reject():
    lib = B.lib()
    qw = lib.w8a8_quantize_weight
    assert qw(None, 4, 64, BUF["aq"], BUF["sa"], None) == NULL
    assert qw(BUF["w"], 0, 64, BUF["aq"], BUF["sa"], None) == SHAPE
    assert qw(BUF["w"], 4, 60, BUF["aq"], BUF["sa"], None) == SHAPE
    assert qw(BUF["w"], 4, B.MAX_K + 8, BUF["aq"], BUF["sa"],
              None) == SHAPE
    assert qw(BUF["w"] + 8, 4, 64, BUF["aq"], BUF["sa"], None) == ALIGN
    assert qw(BUF["w"], 4, 64, BUF["w"] + 256, BUF["sa"], None) == ALIAS
    cs = lib.w8a8_check_scales
    assert cs(None, 4, BUF["out"], None) == NULL
    assert cs(BUF["sw"], -1, BUF["out"], None) == SHAPE
    assert cs(BUF["sw"] + 2, 4, BUF["out"], None) == ALIGN
    assert cs(BUF["sw"], 4, BUF["out"] + 2, None) == ALIGN
    assert cs(BUF["sw"], 4, BUF["sw"] + 8, None) == ALIAS
    sg = lib.w8a8_swiglu_bf16
    assert sg(None, BUF["out"], 2, 64, None) == NULL
    assert sg(BUF["x"], BUF["out"], 2, 12, None) == SHAPE
    assert sg(BUF["x"], BUF["out"], 0, 64, None) == SHAPE
    assert sg(BUF["x"] + 2, BUF["out"], 2, 64, None) == ALIGN
    assert sg(BUF["x"], BUF["x"] + 256, 2, 64, None) == ALIAS
    qs = lib.w8a8_quantize_act_swiglu
    assert qs(BUF["x"], 2, 64, None, BUF["sa"], None) == NULL
    assert qs(BUF["x"], 2, B.GLUE_MAX_K + 8, BUF["aq"], BUF["sa"],
              None) == SHAPE
    assert qs(BUF["x"], 2, 64, BUF["aq"] + 4, BUF["sa"], None) == ALIGN
    assert qs(BUF["x"], 2, 64, BUF["x"] + 128, BUF["sa"], None) == ALIAS


def test_renorm_quantize_rejects():
    lib = B.lib()
    rq = lib.w8a8_pow2_renorm_quantize
    x, y, q, sa = BUF["x"], BUF["out"], BUF["aq"], BUF["sa"]
    assert rq(None, 4, 64, y, q, sa, None) == NULL
    assert rq(x, 4, 64, y, None, sa, None) == NULL
    assert rq(x, 4, 64, y, q, None, None) == NULL
    assert rq(x, 0, 64, y, q, sa, None) == SHAPE
    assert rq(x, 4, 60, y, q, sa, None) == SHAPE
    assert rq(x, 4, B.GLUE_MAX_K + 8, y, q, sa, None) == SHAPE
    assert rq(x + 8, 4, 64, y, q, sa, None) == ALIGN
    assert rq(x, 4, 64, y + 8, q, sa, None) == ALIGN
    assert rq(x, 4, 64, y, q + 4, sa, None) == ALIGN
    assert rq(x, 4, 64, y, q, sa + 2, None) == ALIGN
    assert rq(x, 4, 64, x + 16, q, sa, None) == ALIAS   # y partly over x
    assert rq(x, 4, 64, y, x + 64, sa, None) == ALIAS   # codes over x
    assert rq(x, 4, 64, y, y + 256, sa, None) == ALIAS  # codes over y
    assert rq(x, 4, 64, y, q, q + 64, None) == ALIAS    # scales over codes


def test_no_device_is_reported_without_a_gpu():
    """Valid arguments on a machine without a GPU: the device check, the
    last step before any launch, refuses.  Skipped where a GPU exists
    (there the fake pointers would reach a kernel)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    assert gemm() == DEVICE
    assert quant() == DEVICE


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(B, "LIB_PATH", tmp_path / "missing.so")
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(ImportError):
        B.lib()


def test_build_id_matches_sources(monkeypatch):
    """The library reports the SHA-256 of the sources it was built from;
    the binding refuses to load a build whose sources have changed since."""
    lib = B.lib()
    assert lib.w8a8_build_id().decode() == B._expected_build_id()
    assert not B.build_is_stale()
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "_expected_build_id", lambda: "0" * 64)
    assert B.build_is_stale()
    with pytest.raises(ImportError, match="other sources"):
        B.lib()


def test_library_shares_torchs_hip_runtime():
    """torch's ROCm build carries its own HIP and HSA runtimes.  The binding
    loads the library after torch, so the library's HIP symbols resolve to
    torch's runtime; loaded first (as a stale-build check before any torch
    import once did), it would bring in the system runtime beside torch's,
    and on a GPU the library then saw no device.  In a fresh process:
    exactly one HIP and one HSA runtime are mapped, whatever loads first."""
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from w8a8_int8_gemm_amd import binding as B\n"
        "B.build_is_stale(); B.lib()\n"
        "import torch; torch.zeros(1)\n"
        "maps = open('/proc/self/maps').read().splitlines()\n"
        "for key in ('libamdhip64', 'libhsa-runtime64'):\n"
        "    print(key, sorted({l.split()[-1] for l in maps if key in l}))\n"
    ) % str(ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    import ast
    for line in r.stdout.splitlines():
        key, paths = line.split(" ", 1)
        assert len(ast.literal_eval(paths)) == 1, line  # one of each kind


def test_binding_checks_tensors_before_calling():
    """The wrappers check dtype, shape and device of every tensor before a
    pointer reaches the C ABI (CPU tensors here: refused as not on a GPU)."""
    import torch
    a = torch.zeros((4, 128), dtype=torch.int8)
    with pytest.raises(ValueError):
        B.gemm(a, torch.zeros(4), torch.zeros((128, 128), dtype=torch.int8),
               torch.zeros(128))
    with pytest.raises(ValueError):
        B.quantize_act(torch.zeros((4, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        B.quantize_act(torch.zeros((4, 128), dtype=torch.float32))
    with pytest.raises(TypeError):
        B.pow2_renorm([[1.0]])


def test_mfma_ceiling_library_host_side():
    """The measurement kernel's library (outside the W8A8 ABI) loads,
    counts its operations in closed form and rejects arguments its kernel
    cannot take without launching anything."""
    from w8a8_int8_gemm_amd import build as LB
    lib = ctypes.CDLL(str(LB.CEILING_LIB))
    lib.w8a8_ceiling_ops.restype = ctypes.c_double
    lib.w8a8_ceiling_ops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.w8a8_ceiling_out_len.restype = ctypes.c_int64
    lib.w8a8_ceiling_out_len.argtypes = [ctypes.c_int]
    lib.w8a8_ceiling_run.restype = ctypes.c_int
    lib.w8a8_ceiling_run.argtypes = [ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p]
    # 8 waves x 32 MFMAs of 2*32*32*32 operations per round
    assert lib.w8a8_ceiling_ops(3, 5) == 3 * 8 * 5 * 32 * 65536
    assert lib.w8a8_ceiling_out_len(7) == 7 * 512
    ok = dict(x=BUF["aq"], xr=64, w=BUF["w"], wr=64, K=256, blocks=1,
              iters=1, out=BUF["out"])
    for bad in [dict(x=None), dict(w=None), dict(out=None), dict(xr=31),
                dict(wr=0), dict(K=127), dict(K=136), dict(blocks=0),
                dict(iters=0)]:
        a = {**ok, **bad}
        assert lib.w8a8_ceiling_run(a["x"], a["xr"], a["w"], a["wr"], a["K"],
                                    a["blocks"], a["iters"], a["out"],
                                    None) == 1, bad


def test_noalloc_entry_validates_and_fits_every_plan():
    """w8a8_gemm_noalloc checks its arguments like w8a8_gemm (no workspace
    arguments), and the planner's partial sums fit its scratch for every
    shape: tails of fewer than 256 tiles, skinny split-K grids."""
    lib = B.lib()
    f = lib.w8a8_gemm_noalloc
    ok = dict(aq=BUF["aq"], sa=BUF["sa"], w=BUF["w"], sw=BUF["sw"],
              bias=BUF["bias"], out=BUF["out"], dt=0, M=64, N=5376, K=5376)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["aq"], a["sa"], a["w"], a["sw"], a["bias"], a["out"],
                 a["dt"], a["M"], a["N"], a["K"], None)
    assert call(aq=None) == NULL
    assert call(N=100) == SHAPE
    assert call(dt=7) == OUT_DTYPE
    assert call(sw=BUF["sw"] + 2) == ALIGN
    assert call(out=BUF["w"]) == ALIAS
    import torch
    if torch.cuda.device_count() == 0:
        assert call() == DEVICE
    cap = B.NOALLOC_SCRATCH_BYTES
    import itertools
    worst = 0
    for M, N, K in itertools.product(
            [1, 17, 64, 255, 256, 300, 1100, 4096, 4097, 19077, 37503, 65541],
            [128, 384, 2048, 4096, 5376, 16128, 21504, 28672],
            [128, 640, 5376, 21504, B.MAX_K]):
        worst = max(worst, B.gemm_workspace_bytes(M, N, K))
    assert 0 < worst <= cap
