"""Python binding of libw8a8.so (include/w8a8.h): argument marshalling only.

Torch tensors supply device memory and the current HIP stream; every step
of the computation runs in the library's HIP kernels.  Loading fails loudly
when the shared object is missing: there is no CPU or PyTorch fallback.

BF16 tensors are passed as their bit patterns (the library's uint16 BF16).
"""
from __future__ import annotations

import ctypes
from pathlib import Path

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libw8a8.so"

OUT_BF16, OUT_FP32, OUT_I32 = 0, 1, 2
W8A8_OK = 0
STATUS = {
    0: "W8A8_OK", 1: "W8A8_ERR_NULL", 2: "W8A8_ERR_SHAPE",
    3: "W8A8_ERR_ALIGN", 4: "W8A8_ERR_WORKSPACE", 5: "W8A8_ERR_OUT_DTYPE",
    6: "W8A8_ERR_ALIAS", 7: "W8A8_ERR_DEVICE", 8: "W8A8_ERR_HIP",
}
MAX_K = 130944
GLUE_MAX_K = 90112   # SiLU, renormalization and the fused quantizers

# Every symbol include/w8a8.h declares, with its ctypes signature.
_P, _I64, _SZ, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
SIGNATURES = {
    "w8a8_quantize_act": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "w8a8_quantize_act_silu": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "w8a8_gemm": (_I, [_P, _P, _P, _P, _P, _P, _I, _I64, _I64, _I64, _P,
                       _SZ, _P]),
    "w8a8_linear": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _SZ,
                         _P]),
    "w8a8_gemm_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _I64, _I64,
                               _I64, _P]),
    "w8a8_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "w8a8_gemm_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "w8a8_status_string": (ctypes.c_char_p, [_I]),
    "w8a8_last_hip_error": (_I, []),
    "w8a8_build_id": (ctypes.c_char_p, []),
    "w8a8_silu_bf16": (_I, [_P, _P, _I64, _P]),
    "w8a8_pow2_renorm": (_I, [_P, _P, _I64, _I64, _P]),
    "w8a8_pow2_renorm_quantize": (_I, [_P, _I64, _I64, _P, _P, _P, _P]),
    "w8a8_quantize_weight": (_I, [_P, _I64, _I64, _P, _P, _P]),
    "w8a8_check_scales": (_I, [_P, _I64, _P, _P]),
    "w8a8_swiglu_bf16": (_I, [_P, _P, _I64, _I64, _P]),
    "w8a8_quantize_act_swiglu": (_I, [_P, _I64, _I64, _P, _P, _P]),
}


class W8A8Error(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} "
                         f"({lib().w8a8_status_string(status).decode()})"
                         f"{detail}")


_lib = None


def _load(path):
    # torch first: its ROCm build carries its own HIP runtime, and the
    # library must resolve its HIP symbols to that same runtime (found by
    # its soname once loaded).  Loaded before torch, the library would pull
    # in the system HIP runtime and torch would then load a second one; the
    # library's device calls then fail (no device is visible to it).
    import torch  # noqa: F401
    L = ctypes.CDLL(str(path))
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def _expected_build_id() -> str:
    from . import build as _build
    return _build.source_sha256()


def build_is_stale() -> bool:
    """True when the shared object is missing or was compiled from sources
    other than the ones beside it (read without keeping it loaded)."""
    if not LIB_PATH.exists():
        return True
    if _lib is not None:
        return _lib.w8a8_build_id().decode() != _expected_build_id()
    return _load(LIB_PATH).w8a8_build_id().decode() != _expected_build_id()


def lib():
    """The loaded shared object.  Raises if it has not been built, or if it
    was built from other sources than the ones in the tree (a stale build
    would run old kernels under new code)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m w8a8_int8_gemm_amd.build` (or "
                "__graft_entry__.build()); there is no fallback path")
        L = _load(LIB_PATH)
        got, want = L.w8a8_build_id().decode(), _expected_build_id()
        if got != want:
            raise ImportError(
                f"{LIB_PATH} was built from other sources (build id "
                f"{got[:12]}, sources {want[:12]}): rebuild it with "
                "`python -m w8a8_int8_gemm_amd.build`")
        _lib = L
    return _lib


def _check(fn: str, status: int):
    if status != W8A8_OK:
        detail = ""
        if status == 8:
            detail = f" hipError={lib().w8a8_last_hip_error()}"
        raise W8A8Error(fn, status, detail)


# ---------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(stream, *tensors):
    """Tensors allocated here on torch's current stream but used by kernels
    enqueued on another `stream`: tell the caching allocator, so that it does
    not hand their memory to a later allocation on the current stream while
    those kernels may still read or write it."""
    if stream is None:
        return
    torch = _torch()
    if stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, ndim, name, shape=None):
    """t must be a contiguous tensor of `dtype` with `ndim` dims (and, if
    given, exactly `shape`) on the current GPU: the C ABI takes bare
    pointers, so sizes and devices are checked here."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype or t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} with {ndim} "
                         f"dims, got {t.dtype} {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got "
                         f"{tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} must be on the current GPU "
                         f"(cuda:{torch.cuda.current_device()})")


def quantize_act(x, *, silu: bool = False, out=None, stream=None):
    """x: bf16 [M,K] -> (a_q int8 [M,K], a_scale float32 [M]).
    silu=True applies SiLU (rounded to BF16) before quantizing."""
    torch = _torch()
    _need(x, torch.bfloat16, 2, "x")
    M, K = x.shape
    if out is None:
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
        s = torch.empty((M,), dtype=torch.float32, device=x.device)
    else:
        q, s = out
        _need(q, torch.int8, 2, "out[0]", (M, K))
        _need(s, torch.float32, 1, "out[1]", (M,))
    fn = lib().w8a8_quantize_act_silu if silu else lib().w8a8_quantize_act
    _check("w8a8_quantize_act" + ("_silu" if silu else ""),
           fn(_ptr(x), M, K, _ptr(q), _ptr(s), _stream(stream)))
    if out is None:
        _on_stream(stream, q, s)
    return q, s


def workspace_bytes(M: int, N: int, K: int) -> int:
    """Bytes that serve both linear() and gemm() for this shape."""
    return int(lib().w8a8_workspace_bytes(M, N, K))


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    """Bytes gemm() alone needs (its split-K partial sums)."""
    return int(lib().w8a8_gemm_workspace_bytes(M, N, K))


def _workspace(nbytes, device, given=None):
    torch = _torch()
    if given is not None:
        if not given.is_contiguous() or not given.is_cuda:
            raise ValueError("workspace must be a contiguous GPU tensor")
        return given
    if nbytes == 0:
        return None
    return torch.empty((nbytes,), dtype=torch.uint8, device=device)


def gemm(a_q, a_scale, w_q, w_scale, bias=None, out_dtype=None, *, out=None,
         workspace=None, stream=None):
    """INT8 GEMM + fused epilogue.  out_dtype: torch.bfloat16 (default),
    torch.float32 (epilogue before rounding) or torch.int32 (accumulators).
    """
    torch = _torch()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    codes = {torch.bfloat16: OUT_BF16, torch.float32: OUT_FP32,
             torch.int32: OUT_I32}
    if out_dtype not in codes:
        raise ValueError(f"out_dtype {out_dtype} not supported")
    _need(a_q, torch.int8, 2, "a_q")
    M, K = a_q.shape
    _need(w_q, torch.int8, 2, "w_q")
    N = w_q.shape[0]
    if w_q.shape[1] != K:
        raise ValueError("a_q and w_q disagree on K")
    _need(a_scale, torch.float32, 1, "a_scale", (M,))
    _need(w_scale, torch.float32, 1, "w_scale", (N,))
    if bias is not None:
        _need(bias, torch.bfloat16, 1, "bias", (N,))
    own_out = out is None
    if own_out:
        out = torch.empty((M, N), dtype=out_dtype, device=a_q.device)
    else:
        _need(out, out_dtype, 2, "out", (M, N))
    ws_need = gemm_workspace_bytes(M, N, K)
    ws = _workspace(ws_need, a_q.device, workspace)
    ws_len = 0 if ws is None else ws.numel() * ws.element_size()
    _check("w8a8_gemm", lib().w8a8_gemm(
        _ptr(a_q), _ptr(a_scale), _ptr(w_q), _ptr(w_scale), _ptr(bias),
        _ptr(out), codes[out_dtype], M, N, K, _ptr(ws), ws_len,
        _stream(stream)))
    _on_stream(stream, out if own_out else None,
               ws if workspace is None else None)
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def gemm_noalloc(a_q, a_scale, w_q, w_scale, bias=None, out_dtype=None, *,
                 out, stream=None):
    """gemm() without a workspace: the split-K partial sums go to the
    library's own device scratch (w8a8_gemm_noalloc).  ``out`` must be
    given (nothing is allocated).  Calls that overlap in time on one GPU
    share that scratch: keep them on one stream."""
    torch = _torch()
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    codes = {torch.bfloat16: OUT_BF16, torch.float32: OUT_FP32,
             torch.int32: OUT_I32}
    if out_dtype not in codes:
        raise ValueError(f"out_dtype {out_dtype} not supported")
    _need(a_q, torch.int8, 2, "a_q")
    M, K = a_q.shape
    _need(w_q, torch.int8, 2, "w_q")
    N = w_q.shape[0]
    if w_q.shape[1] != K:
        raise ValueError("a_q and w_q disagree on K")
    _need(a_scale, torch.float32, 1, "a_scale", (M,))
    _need(w_scale, torch.float32, 1, "w_scale", (N,))
    if bias is not None:
        _need(bias, torch.bfloat16, 1, "bias", (N,))
    _need(out, out_dtype, 2, "out", (M, N))
    _check("w8a8_gemm_noalloc", lib().w8a8_gemm_noalloc(
        _ptr(a_q), _ptr(a_scale), _ptr(w_q), _ptr(w_scale), _ptr(bias),
        _ptr(out), codes[out_dtype], M, N, K, _stream(stream)))
    return out


def linear(x, w_q, w_scale, bias=None, *, out=None, workspace=None,
           stream=None):
    """y = bf16(((float)(quant(x) . w_q^T) * sa) * sw + bias)."""
    torch = _torch()
    _need(x, torch.bfloat16, 2, "x")
    M, K = x.shape
    _need(w_q, torch.int8, 2, "w_q")
    N = w_q.shape[0]
    if w_q.shape[1] != K:
        raise ValueError("x and w_q disagree on K")
    _need(w_scale, torch.float32, 1, "w_scale", (N,))
    if bias is not None:
        _need(bias, torch.bfloat16, 1, "bias", (N,))
    own_out = out is None
    if own_out:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _need(out, torch.bfloat16, 2, "out", (M, N))
    ws = _workspace(workspace_bytes(M, N, K), x.device, workspace)
    ws_len = 0 if ws is None else ws.numel() * ws.element_size()
    _check("w8a8_linear", lib().w8a8_linear(
        _ptr(x), _ptr(w_q), _ptr(w_scale), _ptr(bias), _ptr(out), M, N, K,
        _ptr(ws), ws_len, _stream(stream)))
    _on_stream(stream, out if own_out else None,
               ws if workspace is None else None)
    return out


def silu(x, *, out=None, stream=None):
    torch = _torch()
    _need(x, torch.bfloat16, x.dim(), "x")
    y = torch.empty_like(x) if out is None else out
    _need(y, torch.bfloat16, x.dim(), "out", tuple(x.shape))
    _check("w8a8_silu_bf16", lib().w8a8_silu_bf16(
        _ptr(x), _ptr(y), x.numel(), _stream(stream)))
    if out is None:
        _on_stream(stream, y)
    return y


def pow2_renorm(x, *, out=None, stream=None):
    torch = _torch()
    _need(x, torch.bfloat16, 2, "x")
    M, K = x.shape
    y = torch.empty_like(x) if out is None else out
    _need(y, torch.bfloat16, 2, "out", (M, K))
    _check("w8a8_pow2_renorm", lib().w8a8_pow2_renorm(
        _ptr(x), _ptr(y), M, K, _stream(stream)))
    if out is None:
        _on_stream(stream, y)
    return y


def pow2_renorm_quantize(x, *, out=None, stream=None):
    """x: bf16 [M, K] -> (y bf16 [M, K], a_q int8 [M, K], a_scale float32
    [M]): the power-of-two renormalization and the per-token quantization
    of its result, in one pass."""
    torch = _torch()
    _need(x, torch.bfloat16, 2, "x")
    M, K = x.shape
    if out is None:
        y = torch.empty_like(x)
        q = torch.empty((M, K), dtype=torch.int8, device=x.device)
        s = torch.empty((M,), dtype=torch.float32, device=x.device)
    else:
        y, q, s = out
        _need(y, torch.bfloat16, 2, "out[0]", (M, K))
        _need(q, torch.int8, 2, "out[1]", (M, K))
        _need(s, torch.float32, 1, "out[2]", (M,))
    _check("w8a8_pow2_renorm_quantize", lib().w8a8_pow2_renorm_quantize(
        _ptr(x), M, K, _ptr(y), _ptr(q), _ptr(s), _stream(stream)))
    if out is None:
        _on_stream(stream, y, q, s)
    return y, q, s


def quantize_weight(w, *, out=None, stream=None):
    """w: bf16 [N,K] -> (w_q int8 [N,K], w_scale float32 [N]), one scale
    per output channel; all-zero rows get scale 1."""
    torch = _torch()
    _need(w, torch.bfloat16, 2, "w")
    N, K = w.shape
    if out is None:
        q = torch.empty((N, K), dtype=torch.int8, device=w.device)
        s = torch.empty((N,), dtype=torch.float32, device=w.device)
    else:
        q, s = out
        _need(q, torch.int8, 2, "out[0]", (N, K))
        _need(s, torch.float32, 1, "out[1]", (N,))
    _check("w8a8_quantize_weight", lib().w8a8_quantize_weight(
        _ptr(w), N, K, _ptr(q), _ptr(s), _stream(stream)))
    if out is None:
        _on_stream(stream, q, s)
    return q, s


def check_scales(w_scale, *, out=None, stream=None):
    """Device int32 [1]: how many scales are not finite and > 0."""
    torch = _torch()
    _need(w_scale, torch.float32, 1, "w_scale")
    bad = (torch.empty((1,), dtype=torch.int32, device=w_scale.device)
           if out is None else out)
    _need(bad, torch.int32, 1, "out", (1,))
    _check("w8a8_check_scales", lib().w8a8_check_scales(
        _ptr(w_scale), w_scale.numel(), _ptr(bad), _stream(stream)))
    if out is None:
        _on_stream(stream, bad)
    return bad


def swiglu(h, *, out=None, stream=None):
    """h: bf16 [M, 2F] (gate | up) -> bf16 [M, F]."""
    torch = _torch()
    _need(h, torch.bfloat16, 2, "h")
    M, F2 = h.shape
    if F2 % 2:
        raise ValueError("h must have an even width (gate | up)")
    y = (torch.empty((M, F2 // 2), dtype=torch.bfloat16, device=h.device)
         if out is None else out)
    _need(y, torch.bfloat16, 2, "out", (M, F2 // 2))
    _check("w8a8_swiglu_bf16", lib().w8a8_swiglu_bf16(
        _ptr(h), _ptr(y), M, F2 // 2, _stream(stream)))
    if out is None:
        _on_stream(stream, y)
    return y


def quantize_act_swiglu(h, *, out=None, stream=None):
    """h: bf16 [M, 2F] (gate | up) -> (a_q int8 [M,F], a_scale [M]) of
    SwiGLU(h), in one pass."""
    torch = _torch()
    _need(h, torch.bfloat16, 2, "h")
    M, F2 = h.shape
    if F2 % 2:
        raise ValueError("h must have an even width (gate | up)")
    if out is None:
        q = torch.empty((M, F2 // 2), dtype=torch.int8, device=h.device)
        s = torch.empty((M,), dtype=torch.float32, device=h.device)
    else:
        q, s = out
        _need(q, torch.int8, 2, "out[0]", (M, F2 // 2))
        _need(s, torch.float32, 1, "out[1]", (M,))
    _check("w8a8_quantize_act_swiglu", lib().w8a8_quantize_act_swiglu(
        _ptr(h), M, F2 // 2, _ptr(q), _ptr(s), _stream(stream)))
    if out is None:
        _on_stream(stream, q, s)
    return q, s
