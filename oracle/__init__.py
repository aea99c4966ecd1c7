"""CPU oracle of the 4-bit symmetric group quantizer and the quantized product.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library shares
no code with it and never calls it; the product path fails loudly when its own
HIP library is missing instead of falling back to anything here.

The arithmetic lives in ``q4_oracle.c`` (plain C, IEEE fp32 quantization, fp64
product); this module only compiles it with gcc and marshals numpy arrays.
What it follows: QORA-4B forum article (quantization and memory management
section) and QORA-LLM-0.8B model card ("Weight Format", and the Q4 GEMV row of
"AVX-512 SIMD Acceleration"): 4-bit symmetric quantization in groups of 32
with a 16-entry dequantization table.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "q4_oracle.c")
BUILD_DIR = os.path.join(_HERE, "_build")
LIB_PATH = os.path.join(BUILD_DIR, "libq4oracle.so")

OK, ERR_NULL, ERR_SHAPE, ERR_RANGE, ERR_NOMEM = 0, 1, 2, 3, 4

CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c11"]


def compile_oracle(source: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile ``source`` into the shared library ``out`` with gcc."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, "-I", _HERE, source, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str = LIB_PATH):
        self.path = path
        lib = ctypes.CDLL(path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.q4o_f32_to_f16.argtypes = [ctypes.c_float]
        lib.q4o_f32_to_f16.restype = ctypes.c_uint16
        lib.q4o_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.q4o_f16_to_f64.restype = ctypes.c_double
        lib.q4o_quantize.argtypes = [p, i64, i64, p, p]
        lib.q4o_quantize.restype = ctypes.c_int
        lib.q4o_matmul.argtypes = [p, p, p, i64, i64, i64, p, p]
        lib.q4o_matmul_f16.argtypes = [p, p, i64, i64, i64, p, p]
        lib.q4o_matmul_f16.restype = ctypes.c_int
        lib.q4o_matmul.restype = ctypes.c_int
        lib.q4o_threads.argtypes = []
        lib.q4o_threads.restype = ctypes.c_int
        lib.q4o_set_threads.argtypes = [ctypes.c_int]
        lib.q4o_set_threads.restype = None
        self.lib = lib

    def threads(self) -> int:
        return int(self.lib.q4o_threads())

    def set_threads(self, threads: int) -> None:
        """Thread count of later calls (timing only: results never depend on it)."""
        self.lib.q4o_set_threads(int(threads))

    # -- scalar conversions -------------------------------------------------
    def f32_to_f16_bits(self, f: float) -> int:
        return int(self.lib.q4o_f32_to_f16(ctypes.c_float(f)))

    def f16_bits_to_f64(self, h: int) -> float:
        return float(self.lib.q4o_f16_to_f64(ctypes.c_uint16(h)))

    # -- quantizer ----------------------------------------------------------
    def quantize_status(self, w: np.ndarray):
        """Return (status, packed uint8 [n,k/2], scales uint16 [n,k/32])."""
        w = np.ascontiguousarray(w, dtype=np.float32)
        if w.ndim != 2:
            raise ValueError("w must be 2-D [n, k]")
        n, k = w.shape
        packed = np.zeros((n, max(k // 2, 1)), dtype=np.uint8)
        scales = np.zeros((n, max(k // 32, 1)), dtype=np.uint16)
        st = self.lib.q4o_quantize(w.ctypes.data, n, k, packed.ctypes.data,
                                   scales.ctypes.data)
        return st, packed, scales

    def quantize(self, w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        st, packed, scales = self.quantize_status(w)
        if st != OK:
            raise ValueError("oracle quantize failed with status %d" % st)
        return packed, scales

    # -- product ------------------------------------------------------------
    def matmul(self, x_f16: np.ndarray, packed: np.ndarray,
               scales: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """x binary16 [m,k] (np.float16 or uint16 bits) -> (y, bound) fp64 [m,n]."""
        x = np.ascontiguousarray(x_f16)
        if x.dtype == np.float16:
            x = x.view(np.uint16)
        if x.dtype != np.uint16 or x.ndim != 2:
            raise ValueError("x must be 2-D binary16")
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint16)
        m, k = x.shape
        n = packed.shape[0]
        if packed.shape != (n, k // 2) or scales.shape != (n, k // 32):
            raise ValueError("packed/scales shapes do not match x")
        y = np.empty((m, n), dtype=np.float64)
        bound = np.empty((m, n), dtype=np.float64)
        st = self.lib.q4o_matmul(x.ctypes.data, packed.ctypes.data,
                                 scales.ctypes.data, m, n, k, y.ctypes.data,
                                 bound.ctypes.data)
        if st != OK:
            raise ValueError("oracle matmul failed with status %d" % st)
        return y, bound


    def matmul_f16(self, x_f16: np.ndarray, w_f16: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """x binary16 [m,k], w binary16 [n,k] -> (y, bound) fp64 [m,n]."""
        x = np.ascontiguousarray(x_f16)
        w = np.ascontiguousarray(w_f16)
        if x.dtype == np.float16:
            x = x.view(np.uint16)
        if w.dtype == np.float16:
            w = w.view(np.uint16)
        if x.dtype != np.uint16 or w.dtype != np.uint16 or x.ndim != 2 or w.ndim != 2:
            raise ValueError("x and w must be 2-D binary16")
        m, k = x.shape
        n = w.shape[0]
        if w.shape != (n, k):
            raise ValueError("w must be [n, k]")
        y = np.empty((m, n), dtype=np.float64)
        bound = np.empty((m, n), dtype=np.float64)
        st = self.lib.q4o_matmul_f16(x.ctypes.data, w.ctypes.data, m, n, k, y.ctypes.data,
                                     bound.ctypes.data)
        if st != OK:
            raise ValueError("oracle matmul_f16 failed with status %d" % st)
        return y, bound


_default: Optional[Oracle] = None


def get(build_if_missing: bool = True) -> Oracle:
    """The default oracle, compiling it first if no build exists."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            if not build_if_missing:
                raise FileNotFoundError(LIB_PATH)
            compile_oracle()
        _default = Oracle(LIB_PATH)
    return _default


def tolerance(bound: np.ndarray) -> np.ndarray:
    """Allowed |y - y_ref| per output: 1e-3 * sum|x*s*q| + 1e-6."""
    return 1e-3 * bound + 1e-6


def quantize(w):
    return get().quantize(w)


def matmul(x, packed, scales):
    return get().matmul(x, packed, scales)
