"""GPU check of the MFMA-ceiling measurement kernel (libw8a8_ceiling.so,
used only by bench.py): it must perform exactly the integer work it is
timed for.  The sum of a wave's 64 per-lane results is the sum of all
outputs of its 8 accumulators, which has a closed form: for one 32x32x32
product, the sum of all outputs is the dot product of the two fragments'
column sums over that k-step's 32 bytes, so no MFMA output layout is
assumed."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from w8a8_int8_gemm_amd import build as LB

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

TM, TN, KS, WAVES = 2, 4, 4, 8


def lib():
    L = ctypes.CDLL(str(LB.CEILING_LIB))
    vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.w8a8_ceiling_run.restype = ci
    L.w8a8_ceiling_run.argtypes = [vp, i64, vp, i64, i64, ci, ci, vp, vp]
    L.w8a8_ceiling_out_len.restype = i64
    L.w8a8_ceiling_out_len.argtypes = [ci]
    return L


def expected_wave_sums(x, w, blocks, iters):
    xb, wb = x.shape[0] // 32, w.shape[0] // 32
    xs = x.astype(np.int64).reshape(xb, 32, -1).sum(axis=1)  # column sums
    ws = w.astype(np.int64).reshape(wb, 32, -1).sum(axis=1)
    out = []
    for gw in range(blocks * WAVES):
        t = 0
        for i in range(TN):
            for j in range(TM):
                a = ws[(gw * TN + i) % wb, :KS * 32]
                b = xs[(gw * TM + j) % xb, :KS * 32]
                t += int(a @ b)
        out.append(iters * t)
    return np.array(out, np.int64)


@pytest.mark.parametrize("x_rows,w_rows,K,blocks,iters",
                         [(64, 128, 256, 2, 3), (96, 32, 5376, 3, 5)])
def test_ceiling_kernel_work_matches_closed_form(x_rows, w_rows, K, blocks,
                                                 iters):
    print(f"ceiling kernel x {x_rows}x{K}, w {w_rows}x{K}, blocks {blocks}, "
          f"iters {iters}", flush=True)
    rng = np.random.default_rng([x_rows, w_rows, K])
    x = rng.integers(-127, 127, (x_rows, K), endpoint=True, dtype=np.int8)
    w = rng.integers(-127, 127, (w_rows, K), endpoint=True, dtype=np.int8)
    L = lib()
    xd, wd = torch.from_numpy(x).cuda(), torch.from_numpy(w).cuda()
    out = torch.empty((L.w8a8_ceiling_out_len(blocks),), dtype=torch.int32,
                      device="cuda")
    rc = L.w8a8_ceiling_run(xd.data_ptr(), x_rows, wd.data_ptr(), w_rows, K,
                            blocks, iters, out.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    # per-lane sums stay far below 2^31 here, so int64 wave totals are exact
    got = out.cpu().numpy().astype(np.int64).reshape(blocks * WAVES, 64)
    assert np.array_equal(got.sum(axis=1),
                          expected_wave_sums(x, w, blocks, iters))
