"""Python binding of the gfx950 Q4 library (``libq4.so``, C ABI in include/q4.h).

Argument marshalling only: every step of quantization and of the product runs
in the library's HIP kernels.  PyTorch provides device memory and the current
stream.  There is no fallback: if ``libq4.so`` has not been built, or the
current device is not a gfx950, calls raise.

Functions keep the C names:
  q4_quantize(w)                       -> (packed uint8 [n,k/2], scales fp16 [n,k/32])
  q4_gemv(x, packed, scales)           -> y fp32 [m,n]     (1 <= m <= 8)
  q4_gemm(x, packed, scales)           -> y fp32 [m,n]     (any m >= 1)
  q4_gemv_multi(x, [(packed, scales), ...]) -> [y_i fp32 [m,n_i]]  (shared x, <= 8 matrices)
  q4_gemm_multi(x, [(packed, scales), ...]) -> [y_i fp32 [m,n_i]]  (shared x, any m)
  q4_gemv_f16(x, w)                    -> y fp32 [m,n]     (fp16 weights, 1 <= m <= 8)
  q4_gemm_f16(x, w)                    -> y fp32 [m,n]     (fp16 weights, any m)
  q4_gemv_topk(x, packed, scales, topk) -> (values fp32 [m,topk], rows int32 [m,topk])
  q4_gemv_topk_workspace_size(m, n, k) -> bytes of device workspace q4_gemv_topk needs
  q4_gemv_topk_noalloc(x, packed, scales, topk) -> as q4_gemv_topk, scratch held by the library
  q4_status_str(code), q4_abi_version()
Outputs may be passed in (``out=``) to avoid allocation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq4.so")

EXPORTED = ("q4_abi_version", "q4_status_str", "q4_quantize", "q4_gemv", "q4_gemm",
            "q4_gemv_multi", "q4_gemm_multi", "q4_gemv_f16", "q4_gemm_f16", "q4_gemv_topk",
            "q4_gemv_topk_workspace_size", "q4_gemv_topk_noalloc")
(Q4_OK, Q4_ERR_NULL, Q4_ERR_SHAPE, Q4_ERR_ALIGN, Q4_ERR_LAUNCH, Q4_ERR_DEVICE,
 Q4_ERR_WORKSPACE, Q4_ERR_TOO_LARGE) = range(8)
NOALLOC_SCRATCH_BYTES = 16 << 20
TOPK_MAX = 32
GROUP = 32
MULTI_MAX = 8


class Q4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (status %d)" % (fn, q4_status_str(status), status))
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libq4.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libq4.so not built (%s); run python -m q4_group_quantized_amd.build"
                          % path)
    lib = ctypes.CDLL(path)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.q4_abi_version.argtypes = []
    lib.q4_abi_version.restype = ctypes.c_int
    lib.q4_status_str.argtypes = [ctypes.c_int]
    lib.q4_status_str.restype = ctypes.c_char_p
    lib.q4_quantize.argtypes = [p, p, p, i64, i64, p]
    lib.q4_quantize.restype = ctypes.c_int
    for name in ("q4_gemv", "q4_gemm"):
        fn = getattr(lib, name)
        fn.argtypes = [p, p, p, p, i64, i64, i64, p]
        fn.restype = ctypes.c_int
    for name in ("q4_gemv_multi", "q4_gemm_multi"):
        fn = getattr(lib, name)
        fn.argtypes = [p, i64, i64, ctypes.c_int32, p, p, p, p, p]
        fn.restype = ctypes.c_int
    for fn in (lib.q4_gemv_f16, lib.q4_gemm_f16):
        fn.argtypes = [p, p, p, i64, i64, i64, p]
        fn.restype = ctypes.c_int
    lib.q4_gemv_topk_workspace_size.argtypes = [i64, i64, i64]
    lib.q4_gemv_topk_workspace_size.restype = ctypes.c_size_t
    lib.q4_gemv_topk.argtypes = [p, p, p, i64, i64, i64, ctypes.c_int32, p, p, p,
                                 ctypes.c_size_t, p]
    lib.q4_gemv_topk.restype = ctypes.c_int
    lib.q4_gemv_topk_noalloc.argtypes = [p, p, p, i64, i64, i64, ctypes.c_int32, p, p, p]
    lib.q4_gemv_topk_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


def q4_abi_version() -> int:
    return int(load().q4_abi_version())


def q4_status_str(status: int) -> str:
    return load().q4_status_str(int(status)).decode()


def _stream(stream, device) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _check(fn: str, status: int) -> None:
    if status != Q4_OK:
        raise Q4Error(fn, status)


def _require(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def q4_quantize(w, out: Optional[Tuple] = None, stream=None):
    """fp32 [n, k] device tensor -> (packed uint8 [n, k/2], scales fp16 [n, k/32])."""
    import torch
    _require(w, torch.float32, "w")
    if w.dim() != 2:
        raise ValueError("w must be 2-D [n, k]")
    n, k = w.shape
    if out is None:
        packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
        scales = torch.empty((n, k // GROUP), dtype=torch.float16, device=w.device)
    else:
        packed, scales = out
    with torch.cuda.device(w.device):
        st = load().q4_quantize(w.data_ptr(), packed.data_ptr(), scales.data_ptr(), n, k,
                                _stream(stream, w.device))
    _check("q4_quantize", st)
    return packed, scales


def _product(name, x, packed, scales, out, stream):
    import torch
    _require(x, torch.float16, "x")
    _require(packed, torch.uint8, "packed")
    _require(scales, torch.float16, "scales")
    if x.dim() != 2 or packed.dim() != 2 or scales.dim() != 2:
        raise ValueError("x, packed and scales must be 2-D")
    m, k = x.shape
    n = packed.shape[0]
    if packed.shape[1] * 2 != k or tuple(scales.shape) != (n, k // GROUP):
        raise ValueError("shapes disagree: x %s packed %s scales %s"
                         % (tuple(x.shape), tuple(packed.shape), tuple(scales.shape)))
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=x.device)
    if out is not None:
        _require(y, torch.float32, "out")
        if tuple(y.shape) != (m, n):
            raise ValueError("out must be [m, n]")
    with torch.cuda.device(x.device):
        st = getattr(load(), name)(x.data_ptr(), packed.data_ptr(), scales.data_ptr(),
                                   y.data_ptr(), m, n, k, _stream(stream, x.device))
    _check(name, st)
    return y


def q4_gemv(x, packed, scales, out=None, stream=None):
    """Decode product, 1 <= m <= 8: y[m, n] = x[m, k] . dequant(packed, scales)^T."""
    return _product("q4_gemv", x, packed, scales, out, stream)


def q4_gemm(x, packed, scales, out=None, stream=None):
    """Prefill product for any m >= 1 (tuned for m >= 16)."""
    return _product("q4_gemm", x, packed, scales, out, stream)


def q4_gemv_multi(x, mats, out=None, stream=None):
    """Decode products of several matrices over the same x in one call.

    mats: sequence of (packed, scales) pairs with the same k; returns the list
    of y_i [m, n_i] (or fills ``out``, a list of fp32 [m, n_i] tensors)."""
    return _multi("q4_gemv_multi", x, mats, out, stream)


def q4_gemm_multi(x, mats, out=None, stream=None):
    """Prefill products of several matrices over the same token batch in one launch."""
    return _multi("q4_gemm_multi", x, mats, out, stream)


def _multi(name, x, mats, out, stream):
    import torch
    _require(x, torch.float16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [m, k]")
    m, k = x.shape
    count = len(mats)
    if out is not None and len(out) != count:
        raise ValueError("out must hold one tensor per matrix")
    ys = []
    for i, (packed, scales) in enumerate(mats):
        _require(packed, torch.uint8, "packed[%d]" % i)
        _require(scales, torch.float16, "scales[%d]" % i)
        n = packed.shape[0]
        if packed.dim() != 2 or packed.shape[1] * 2 != k or tuple(scales.shape) != (n, k // GROUP):
            raise ValueError("matrix %d: shapes disagree with x %s" % (i, tuple(x.shape)))
        if out is None:
            ys.append(torch.empty((m, n), dtype=torch.float32, device=x.device))
        else:
            _require(out[i], torch.float32, "out[%d]" % i)
            if tuple(out[i].shape) != (m, n):
                raise ValueError("out[%d] must be [m, n]" % i)
            ys.append(out[i])
    ptrs = ctypes.c_void_p * max(count, 1)
    packed_a = ptrs(*[p.data_ptr() for p, _ in mats])
    scales_a = ptrs(*[s.data_ptr() for _, s in mats])
    y_a = ptrs(*[y.data_ptr() for y in ys])
    n_a = (ctypes.c_int64 * max(count, 1))(*[p.shape[0] for p, _ in mats])
    with torch.cuda.device(x.device):
        st = getattr(load(), name)(x.data_ptr(), m, k, count, packed_a, scales_a, y_a, n_a,
                                   _stream(stream, x.device))
    _check(name, st)
    return ys


def q4_gemv_f16(x, w, out=None, stream=None):
    """Decode product with fp16 weights: y[m, n] = x[m, k] . w[n, k]^T, 1 <= m <= 8."""
    return _f16("q4_gemv_f16", x, w, out, stream)


def q4_gemm_f16(x, w, out=None, stream=None):
    """Prefill product with fp16 weights: q4_gemv_f16 for any m >= 1."""
    return _f16("q4_gemm_f16", x, w, out, stream)


def _f16(name, x, w, out, stream):
    import torch
    _require(x, torch.float16, "x")
    _require(w, torch.float16, "w")
    if x.dim() != 2 or w.dim() != 2 or w.shape[1] != x.shape[1]:
        raise ValueError("x [m, k] and w [n, k] required, got %s and %s"
                         % (tuple(x.shape), tuple(w.shape)))
    m, k = x.shape
    n = w.shape[0]
    y = out if out is not None else torch.empty((m, n), dtype=torch.float32, device=x.device)
    if out is not None:
        _require(y, torch.float32, "out")
        if tuple(y.shape) != (m, n):
            raise ValueError("out must be [m, n]")
    with torch.cuda.device(x.device):
        st = getattr(load(), name)(x.data_ptr(), w.data_ptr(), y.data_ptr(), m, n, k,
                                   _stream(stream, x.device))
    _check(name, st)
    return y


def q4_gemv_topk_workspace_size(m: int, n: int, k: int) -> int:
    """Bytes of device workspace q4_gemv_topk needs on the current device (0: invalid)."""
    return int(load().q4_gemv_topk_workspace_size(m, n, k))


def q4_gemv_topk(x, packed, scales, topk, workspace=None, out=None, stream=None):
    """The topk largest logits of x . dequant(W)^T per token and their rows.

    Returns (values fp32 [m, topk], rows int32 [m, topk]), largest first, equal
    values by smaller row.  `workspace` (uint8 device tensor) is allocated when
    not given; `out` may pass the (values, rows) tensors."""
    import torch
    _require(x, torch.float16, "x")
    _require(packed, torch.uint8, "packed")
    _require(scales, torch.float16, "scales")
    m, k = x.shape
    n = packed.shape[0]
    if packed.shape[1] * 2 != k or tuple(scales.shape) != (n, k // GROUP):
        raise ValueError("shapes disagree: x %s packed %s scales %s"
                         % (tuple(x.shape), tuple(packed.shape), tuple(scales.shape)))
    with torch.cuda.device(x.device):
        need = q4_gemv_topk_workspace_size(m, n, k)
        if workspace is None:
            workspace = torch.empty(max(need, 1) + 256, dtype=torch.uint8, device=x.device)
        _require(workspace, torch.uint8, "workspace")
        ws_ptr = workspace.data_ptr()
        pad = (-ws_ptr) % 256
        ws_bytes = workspace.numel() - pad if workspace.numel() >= pad else 0
        if out is None:
            values = torch.empty((m, topk), dtype=torch.float32, device=x.device)
            rows = torch.empty((m, topk), dtype=torch.int32, device=x.device)
        else:
            values, rows = out
            _require(values, torch.float32, "values")
            _require(rows, torch.int32, "rows")
        st = load().q4_gemv_topk(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), m, n, k,
                                 int(topk), values.data_ptr(), rows.data_ptr(), ws_ptr + pad,
                                 ws_bytes, _stream(stream, x.device))
    _check("q4_gemv_topk", st)
    return values, rows


def q4_gemv_topk_noalloc(x, packed, scales, topk, out=None, stream=None):
    """q4_gemv_topk without a workspace: the library's own scratch buffer
    (NOALLOC_SCRATCH_BYTES per device) serves the call, so the C call
    allocates nothing.  Calls that overlap in time on one device race on that
    buffer.  `out` may pass the (values fp32 [m, topk], rows int32 [m, topk])
    tensors; otherwise they are allocated here with torch."""
    import torch
    _require(x, torch.float16, "x")
    _require(packed, torch.uint8, "packed")
    _require(scales, torch.float16, "scales")
    m, k = x.shape
    n = packed.shape[0]
    if packed.shape[1] * 2 != k or tuple(scales.shape) != (n, k // GROUP):
        raise ValueError("shapes disagree: x %s packed %s scales %s"
                         % (tuple(x.shape), tuple(packed.shape), tuple(scales.shape)))
    if out is None:
        values = torch.empty((m, topk), dtype=torch.float32, device=x.device)
        rows = torch.empty((m, topk), dtype=torch.int32, device=x.device)
    else:
        values, rows = out
        _require(values, torch.float32, "values")
        _require(rows, torch.int32, "rows")
    with torch.cuda.device(x.device):
        st = load().q4_gemv_topk_noalloc(x.data_ptr(), packed.data_ptr(), scales.data_ptr(), m,
                                         n, k, int(topk), values.data_ptr(), rows.data_ptr(),
                                         _stream(stream, x.device))
    _check("q4_gemv_topk_noalloc", st)
    return values, rows
