"""w8a8_gemm_noalloc (the GEMM entry point that allocates nothing: its
split-K partial sums live in the library's device scratch) against
w8a8_gemm with a caller's workspace, bit for bit, on two calls in a row,
the second with a smaller input; outputs sit between guard bytes."""
from __future__ import annotations

import numpy as np
import pytest

from w8a8_int8_gemm_amd import binding as B
from w8a8_int8_gemm_amd import block as BL

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

GUARD = 4096


def inputs(M, N, K, seed):
    g = np.random.default_rng([seed, M, N, K])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    a = t(g.integers(-128, 128, (M, K), dtype=np.int8))
    w = t(g.integers(-128, 128, (N, K), dtype=np.int8))
    sa = t(np.exp(g.normal(-4, 2, M)).astype(np.float32))
    sw = t(np.exp(g.normal(-6, 0.3, N)).astype(np.float32))
    bias = t(g.normal(0, 0.02, N).astype(np.float32)).to(torch.bfloat16)
    return a, sa, w, sw, bias


def guarded(M, N, dtype):
    n = M * N * torch.empty((), dtype=dtype).element_size()
    raw = torch.full((GUARD + n + GUARD,), 0xA5, dtype=torch.uint8,
                     device="cuda")
    return raw, raw[GUARD:GUARD + n].view(dtype).view(M, N)


# First a large-tile shape with a split tail (partial sums of 48 tail-tile
# slices in the scratch), then a smaller skinny shape (split-K over the
# whole output), then a shape with no split at all.
SHAPES = [(4097, 4096, 1664), (128, 5376, 5376), (300, 384, 640)]


def test_noalloc_equals_gemm_on_consecutive_calls():
    assert B.gemm_workspace_bytes(*SHAPES[0]) > \
        B.gemm_workspace_bytes(*SHAPES[1]) > 0
    for i, (M, N, K) in enumerate(SHAPES):
        print(f"gemm_noalloc call {i}: M={M} N={N} K={K}", flush=True)
        args = inputs(M, N, K, 40 + i)
        for dt in (torch.bfloat16, torch.int32, torch.float32):
            want = B.gemm(*args, out_dtype=dt)
            raw, out = guarded(M, N, dt)
            B.gemm_noalloc(*args, out_dtype=dt, out=out)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.uint8), want.view(torch.uint8)), \
                (M, N, K, dt)
            head, tail = raw[:GUARD], raw[-GUARD:]
            assert bool((head == 0xA5).all()) and bool((tail == 0xA5).all())


def test_noalloc_rejects_like_gemm():
    a, sa, w, sw, bias = inputs(64, 256, 256, 7)
    out = torch.empty((64, 256), dtype=torch.bfloat16, device="cuda")
    # an output overlapping an input, or a bad shape, is refused before any
    # launch
    lib = B.lib()
    rc = lib.w8a8_gemm_noalloc(a.data_ptr(), sa.data_ptr(), w.data_ptr(),
                               sw.data_ptr(), bias.data_ptr(), a.data_ptr(),
                               B.OUT_BF16, 64, 256, 256, None)
    assert rc == 6  # W8A8_ERR_ALIAS
    rc = lib.w8a8_gemm_noalloc(a.data_ptr(), sa.data_ptr(), w.data_ptr(),
                               sw.data_ptr(), bias.data_ptr(), out.data_ptr(),
                               B.OUT_BF16, 64, 200, 256, None)
    assert rc == 2  # W8A8_ERR_SHAPE


def test_noalloc_replays_in_a_captured_graph():
    """The callers this entry point is for include code under HIP graph
    capture: a captured split-tail call (its partial sums in the scratch),
    replayed three times with eager calls between the replays that write
    the same scratch for another shape, matches the eager w8a8_gemm on
    every replay."""
    M, N, K = SHAPES[0]
    args = inputs(M, N, K, 77)
    want = B.gemm(*args)
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    B.gemm_noalloc(*args, out=out)  # one-time set-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.gemm_noalloc(*args, out=out)
    Mo, No, Ko = SHAPES[1]
    other = inputs(Mo, No, Ko, 78)
    other_out = torch.empty((Mo, No), dtype=torch.bfloat16, device="cuda")
    for r in range(3):
        print(f"graph replay {r}", flush=True)
        out.zero_()
        B.gemm_noalloc(*other, out=other_out)  # dirties the scratch
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), r
