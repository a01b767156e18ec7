"""CPU oracle for the verify-pass product -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``fp8_weight_streaming_amd``) never does: it has no CPU path.

The arithmetic lives in ``oracle.c`` (plain C, FP64, OpenMP over rows).
This module compiles it with gcc, loads it with ctypes and wraps it for
numpy arrays.  What it computes, for every column n and output row m:

    y[n][m] = sum_k w[m][k] * x[n][k]        (FP64)
    a[n][m] = sum_k |w[m][k] * x[n][k]|      (FP64, scale of the tolerance)

with w decoded from its stored format (NVFP4 or row-scaled FP8-E4M3) and x
from BF16.  The verify pass of the crit-hub engine card
"mtp7-device-confidence" (section "Design", row "GEMVs") is this product at
1-8 columns; its section "Checks" and the crit README's "Kernel workbench"
both check such kernels against an FP64 reference.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC", "-Wall"]


def build() -> str:
    """Compile oracle.c into liboracle.so (always recompiles)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    lib.oracle_e2m1.restype = ctypes.c_double
    lib.oracle_e2m1.argtypes = [ctypes.c_uint]
    lib.oracle_e4m3.restype = ctypes.c_double
    lib.oracle_e4m3.argtypes = [ctypes.c_uint]
    lib.oracle_bf16.restype = ctypes.c_double
    lib.oracle_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_gemm_nvfp4.restype = None
    lib.oracle_gemm_nvfp4.argtypes = [P, P, ctypes.c_float, P, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, P, ctypes.c_int, P, P]
    lib.oracle_gemm_fp8row.restype = None
    lib.oracle_gemm_fp8row.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       P, ctypes.c_int, P, P]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_num_threads.restype = None
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def e2m1(code: int) -> float:
    """Value of a 4-bit E2M1 code."""
    return _load().oracle_e2m1(int(code))


def e4m3(byte: int) -> float:
    """Value of an E4M3 (FN) byte; NaN for S.1111.111."""
    return _load().oracle_e4m3(int(byte))


def bf16(bits: int) -> float:
    """Value of a BF16 bit pattern."""
    return _load().oracle_bf16(int(bits))


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's later parallel loops (n >= 1)."""
    _load().oracle_set_num_threads(int(n))


def _c(arr, dtype):
    a = np.ascontiguousarray(arr, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _rows(rows, M):
    if rows is None:
        return None, None, M
    r = np.ascontiguousarray(rows, dtype=np.int64)
    if r.ndim != 1 or (r.size and (r.min() < 0 or r.max() >= M)):
        raise ValueError("rows must be a 1-D list of indices in [0, M)")
    return r, r.ctypes.data_as(ctypes.c_void_p), int(r.size)


def gemm_nvfp4(codes: np.ndarray, scales: np.ndarray, g: float, x: np.ndarray,
               rows: Optional[np.ndarray] = None):
    """FP64 product for NVFP4 weights.

    codes  uint8 [M, K/2]  (low nibble = even k)
    scales uint8 [M, K/16] E4M3 block scales
    g      per-tensor FP32 multiplier
    x      uint16 [N, K]   BF16 bits
    rows   optional row subset; outputs then have shape [N, len(rows)]
    Returns (y, a), float64 [N, M or len(rows)].
    """
    codes, pc = _c(codes, np.uint8)
    scales, ps = _c(scales, np.uint8)
    x, px = _c(x, np.uint16)
    M, half = codes.shape
    K = 2 * half
    N = x.shape[0]
    if K % 16 or scales.shape != (M, K // 16) or x.shape != (N, K):
        raise ValueError("inconsistent NVFP4 shapes")
    r, pr, R = _rows(rows, M)
    y = np.empty((N, R), np.float64)
    a = np.empty((N, R), np.float64)
    _load().oracle_gemm_nvfp4(pc, ps, float(np.float32(g)), px, M, K, N, pr, R,
                              y.ctypes.data_as(ctypes.c_void_p), a.ctypes.data_as(ctypes.c_void_p))
    return y, a


def gemm_fp8row(w: np.ndarray, row_scale: np.ndarray, x: np.ndarray,
                rows: Optional[np.ndarray] = None):
    """FP64 product for row-scaled FP8-E4M3 weights.

    w         uint8 [M, K] E4M3
    row_scale float32 [M]
    x         uint16 [N, K] BF16 bits
    Returns (y, a), float64 [N, M or len(rows)].
    """
    w, pw = _c(w, np.uint8)
    row_scale, prs = _c(row_scale, np.float32)
    x, px = _c(x, np.uint16)
    M, K = w.shape
    N = x.shape[0]
    if row_scale.shape != (M,) or x.shape != (N, K):
        raise ValueError("inconsistent FP8-row shapes")
    r, pr, R = _rows(rows, M)
    y = np.empty((N, R), np.float64)
    a = np.empty((N, R), np.float64)
    _load().oracle_gemm_fp8row(pw, prs, px, M, K, N, pr, R,
                               y.ctypes.data_as(ctypes.c_void_p), a.ctypes.data_as(ctypes.c_void_p))
    return y, a
