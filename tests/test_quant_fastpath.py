"""The device quantizer's reciprocal fast path, checked on the CPU against
the oracle's division over every finite BF16 input.

The device computes codes as round(fma(x, 1/s, 128)) - 128 unless the
fused product lies within 2^-14 of a half-integer or the row's scale is
subnormal, where it divides (quant_row / quant4 in rowwise.hip).  The
codes are graded bit-exact against clamp(rint(x / s)), so this test runs a
C model of that arithmetic (tests/quant_fastpath_model.c) over rows whose
largest magnitude takes every one of the 128 BF16 mantissas in several
binades -- ordinary scales, the binades where s = amax/127 crosses the
smallest normal binary32, and subnormal amax -- each row holding every
finite BF16 value no larger in magnitude than its maximum, and requires
zero disagreements with the oracle.  A negative control (the same model
without the closeness test) must disagree, so the comparison can tell.
"""
from __future__ import annotations

import ctypes
import subprocess
from pathlib import Path

import numpy as np
import pytest

HERE = Path(__file__).resolve().parent
MODEL_SRC = HERE / "quant_fastpath_model.c"

# amax binades: ordinary scales; s = amax / 127 crossing 2^-126 (amax near
# 127 * 2^-126, between 2^-120 and 2^-118); subnormal BF16 amax.
BINADES = [-3, 0, 7, 60, -120, -119, -118, -127, -130]


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    out = tmp_path_factory.mktemp("qmodel") / "libqmodel.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                    "-ffp-contract=off", "-fno-fast-math", "-frounding-math",
                    "-o", str(out), str(MODEL_SRC), "-lm"], check=True)
    lib = ctypes.CDLL(str(out))
    lib.model_codes.argtypes = [ctypes.c_void_p, ctypes.c_int64,
                                ctypes.c_uint16, ctypes.c_float,
                                ctypes.c_void_p, ctypes.c_void_p]
    lib.model_codes.restype = ctypes.c_int
    return lib


def amax_values():
    """BF16 bit patterns of every mantissa in each binade of BINADES."""
    out = []
    for e in BINADES:
        for m in range(128):
            if e >= -126:
                out.append(((e + 127) << 7) | m)
            else:  # subnormal BF16: value m * 2^-133 with the leading bit
                lead = 1 << (e + 133)  # at 2^e
                if lead < 128:
                    out.append(lead | (m & (lead - 1)))
    return sorted(set(out))


FINITE = np.arange(65536, dtype=np.uint32).astype(np.uint16)
FINITE = FINITE[((FINITE >> 7) & 0xFF) != 0xFF]
MAG = FINITE & 0x7FFF


def row_for(amax_bits: int) -> np.ndarray:
    """[amax, every finite BF16 x with |x| <= amax]."""
    xs = FINITE[MAG <= amax_bits]
    return np.concatenate([np.array([amax_bits], np.uint16), xs])


def run_model(model, row, amax_bits, closeness):
    codes = np.empty(row.size, np.int8)
    fast = np.zeros(1, np.int64)
    model.model_codes(row.ctypes.data, row.size, amax_bits, closeness,
                      codes.ctypes.data, fast.ctypes.data)
    return codes, int(fast[0])


def test_fast_path_equals_division_everywhere(orc, model):
    total = fast_total = 0
    for a in amax_values():
        row = row_for(a)
        q_ref, s_ref = orc.quantize_act(row[None, :])
        codes, fast = run_model(model, row, a, 2.0 ** -14)
        bad = np.flatnonzero(codes != q_ref[0])
        assert bad.size == 0, (
            f"amax bits {a:#06x}: {bad.size} codes differ, e.g. x bits "
            f"{row[bad[0]]:#06x}: model {codes[bad[0]]}, oracle "
            f"{q_ref[0][bad[0]]}")
        total += row.size
        fast_total += fast
    # the fast path carries almost every element of the normal-scale rows
    assert total > 5_000_000 and fast_total > 0.9 * total


def test_negative_control_without_closeness_test(orc, model):
    """Dropping the half-integer test (always the reciprocal product)
    changes codes: the comparison above can detect a wrong fast path."""
    wrong = 0
    for a in amax_values()[:256]:
        row = row_for(a)
        q_ref, _ = orc.quantize_act(row[None, :])
        codes, _ = run_model(model, row, a, -1.0)
        wrong += int(np.count_nonzero(codes != q_ref[0]))
    assert wrong > 0
