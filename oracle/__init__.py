"""CPU oracle of the W8A8 INT8 projection -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package.  It wraps the plain C reference in
``w8a8_oracle.c`` (built by ``oracle/build.py``) with numpy marshalling;
no arithmetic of the method happens in Python here.

Arrays: BF16 values travel as ``uint16`` bit patterns, INT8 as ``int8``,
scales as ``float32``, accumulators as ``int32``; all C-contiguous and
row-major.  The oracle's sources are cited in ``w8a8_oracle.h``.

``Oracle(path)`` wraps any build of the C file (the mutation tests load
deliberately broken builds through it); the module-level functions use
the default build ``oracle/libw8a8_oracle.so``.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
# W8A8_ORACLE_LIB names another build of the same source (the sanitizer
# test runs the pins against a -fsanitize=undefined build this way).
LIB_PATH = Path(os.environ.get("W8A8_ORACLE_LIB",
                               _HERE / "libw8a8_oracle.so"))

_ERRORS = {
    1: "NULL pointer",
    2: "size out of range",
    3: "non-finite activation",
    4: "weight scale not finite or not > 0",
    5: "accumulator outside INT32",
}


class OracleError(RuntimeError):
    def __init__(self, what: str, code: int):
        super().__init__(f"{what}: {_ERRORS.get(code, code)}")
        self.code = code


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


class Oracle:
    def __init__(self, path: Path | str = LIB_PATH):
        path = Path(path)
        if not path.exists():
            raise FileNotFoundError(
                f"{path} is missing; run oracle/build.py (or "
                "__graft_entry__.build()) first")
        lib = ctypes.CDLL(str(path))
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        sigs = {
            "orc_quantize_act": [P, I64, I64, P, P],
            "orc_quantize_weight": [P, I64, I64, P, P],
            "orc_check_scales": [P, I64, P],
            "orc_gemm_i32": [P, P, I64, I64, I64, P],
            "orc_epilogue": [P, P, P, P, I64, I64, P, P],
            "orc_linear": [P, P, P, P, I64, I64, I64, P],
            "orc_silu_bf16": [P, I64, P],
            "orc_swiglu_bf16": [P, I64, I64, P],
            "orc_pow2_renorm": [P, I64, I64, P],
            "orc_num_threads": [],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f32.restype = ctypes.c_float
        lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.orc_f32_to_bf16.restype = ctypes.c_uint16
        lib.orc_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.orc_f64_to_bf16.restype = ctypes.c_uint16
        self.lib = lib
        self.path = path

    @staticmethod
    def _check(rc: int, what: str):
        if rc != 0:
            raise OracleError(what, rc)

    def num_threads(self) -> int:
        return int(self.lib.orc_num_threads())

    def quantize_act(self, x_bf16: np.ndarray):
        """x: uint16 [M,K] BF16 bits -> (q int8 [M,K], sa float32 [M])."""
        x = _c(x_bf16, np.uint16)
        M, K = x.shape
        q = np.empty((M, K), np.int8)
        sa = np.empty(M, np.float32)
        self._check(self.lib.orc_quantize_act(_ptr(x), M, K, _ptr(q),
                                              _ptr(sa)), "quantize_act")
        return q, sa

    def quantize_weight(self, w_bf16: np.ndarray):
        """w: uint16 [N,K] BF16 bits -> (q int8 [N,K], sw float32 [N])."""
        w = _c(w_bf16, np.uint16)
        N, K = w.shape
        q = np.empty((N, K), np.int8)
        sw = np.empty(N, np.float32)
        self._check(self.lib.orc_quantize_weight(_ptr(w), N, K, _ptr(q),
                                                 _ptr(sw)), "quantize_weight")
        return q, sw

    def check_scales(self, sw: np.ndarray) -> int:
        """Number of scales that are not finite and > 0."""
        sw = _c(sw, np.float32)
        bad = np.zeros(1, np.int64)
        self._check(self.lib.orc_check_scales(_ptr(sw), sw.size, _ptr(bad)),
                    "check_scales")
        return int(bad[0])

    def gemm_i32(self, a: np.ndarray, w: np.ndarray) -> np.ndarray:
        """a int8 [M,K], w int8 [N,K] -> acc int32 [M,N]."""
        a = _c(a, np.int8)
        w = _c(w, np.int8)
        M, K = a.shape
        N, K2 = w.shape
        if K != K2:
            raise ValueError("K mismatch")
        acc = np.empty((M, N), np.int32)
        self._check(self.lib.orc_gemm_i32(_ptr(a), _ptr(w), M, N, K,
                                          _ptr(acc)), "gemm_i32")
        return acc

    def epilogue(self, acc, sa, sw, bias=None):
        """-> (y_f32 float32 [M,N], y_bf16 uint16 [M,N])."""
        acc = _c(acc, np.int32)
        sa = _c(sa, np.float32)
        sw = _c(sw, np.float32)
        bias = None if bias is None else _c(bias, np.uint16)
        M, N = acc.shape
        if sa.shape != (M,) or sw.shape != (N,) or (
                bias is not None and bias.shape != (N,)):
            raise ValueError("scale/bias shape mismatch")
        yf = np.empty((M, N), np.float32)
        yb = np.empty((M, N), np.uint16)
        self._check(self.lib.orc_epilogue(_ptr(acc), _ptr(sa), _ptr(sw),
                                          _ptr(bias), M, N, _ptr(yf),
                                          _ptr(yb)), "epilogue")
        return yf, yb

    def linear(self, x_bf16, w, sw, bias=None) -> np.ndarray:
        """x uint16 [M,K], w int8 [N,K], sw float32 [N], bias uint16 [N]
        or None -> y uint16 [M,N] (BF16 bits)."""
        x = _c(x_bf16, np.uint16)
        w = _c(w, np.int8)
        sw = _c(sw, np.float32)
        bias = None if bias is None else _c(bias, np.uint16)
        M, K = x.shape
        N, K2 = w.shape
        if K != K2 or sw.shape != (N,):
            raise ValueError("shape mismatch")
        y = np.empty((M, N), np.uint16)
        self._check(self.lib.orc_linear(_ptr(x), _ptr(w), _ptr(sw),
                                        _ptr(bias), M, N, K, _ptr(y)),
                    "linear")
        return y

    def silu_bf16(self, x_bf16) -> np.ndarray:
        x = _c(x_bf16, np.uint16)
        y = np.empty_like(x)
        self._check(self.lib.orc_silu_bf16(_ptr(x), x.size, _ptr(y)),
                    "silu_bf16")
        return y

    def swiglu_bf16(self, h_bf16) -> np.ndarray:
        """h uint16 [M, 2F] (gate | up) -> y uint16 [M, F]."""
        h = _c(h_bf16, np.uint16)
        M, F2 = h.shape
        if F2 % 2:
            raise ValueError("odd width")
        y = np.empty((M, F2 // 2), np.uint16)
        self._check(self.lib.orc_swiglu_bf16(_ptr(h), M, F2 // 2, _ptr(y)),
                    "swiglu_bf16")
        return y

    def pow2_renorm(self, x_bf16) -> np.ndarray:
        x = _c(x_bf16, np.uint16)
        M, K = x.shape
        y = np.empty_like(x)
        self._check(self.lib.orc_pow2_renorm(_ptr(x), M, K, _ptr(y)),
                    "pow2_renorm")
        return y

    # Scalar conversions, element by element (slow; for tests).
    def f32_to_bf16(self, values) -> np.ndarray:
        v = np.asarray(values, np.float32).ravel()
        f = self.lib.orc_f32_to_bf16
        return np.array([f(float(t)) for t in v], np.uint16)

    def f64_to_bf16(self, values) -> np.ndarray:
        v = np.asarray(values, np.float64).ravel()
        f = self.lib.orc_f64_to_bf16
        return np.array([f(float(t)) for t in v], np.uint16)

    def bf16_to_f32(self, bits) -> np.ndarray:
        b = np.asarray(bits, np.uint16).ravel()
        f = self.lib.orc_bf16_to_f32
        return np.array([f(int(t)) for t in b], np.float32)


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(LIB_PATH)
    return _default


def quantize_act(x_bf16):
    return default().quantize_act(x_bf16)


def quantize_weight(w_bf16):
    return default().quantize_weight(w_bf16)


def check_scales(sw):
    return default().check_scales(sw)


def swiglu_bf16(h_bf16):
    return default().swiglu_bf16(h_bf16)


def gemm_i32(a, w):
    return default().gemm_i32(a, w)


def epilogue(acc, sa, sw, bias=None):
    return default().epilogue(acc, sa, sw, bias)


def linear(x_bf16, w, sw, bias=None):
    return default().linear(x_bf16, w, sw, bias)


def silu_bf16(x_bf16):
    return default().silu_bf16(x_bf16)


def pow2_renorm(x_bf16):
    return default().pow2_renorm(x_bf16)


def num_threads() -> int:
    return default().num_threads()
