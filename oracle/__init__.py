"""ctypes front end of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg are the only callers.  The product path (gemm_q4_q5_amd) never
imports this package, and this package never imports the product.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

Q4_K, Q5_K, Q6_K, NVFP4, FP8 = 12, 13, 14, 1001, 1002


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc: plain -O2, OpenMP, no fast-math, no FMA contraction."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off",
                               "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=False)
        L = ctypes.CDLL(LIB)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.oracle_fp16.argtypes, L.oracle_fp16.restype = [ctypes.c_uint16], ctypes.c_double
        L.oracle_e4m3.argtypes, L.oracle_e4m3.restype = [ctypes.c_uint8], ctypes.c_double
        L.oracle_e2m1.argtypes, L.oracle_e2m1.restype = [ctypes.c_uint8], ctypes.c_double
        L.oracle_bf16.argtypes, L.oracle_bf16.restype = [ctypes.c_uint16], ctypes.c_double
        L.oracle_row_bytes.argtypes, L.oracle_row_bytes.restype = [i32, i64], i64
        L.oracle_dequant.argtypes = [i32, p, p, i64, i64, i64, i64, p]
        L.oracle_dequant.restype = ctypes.c_int
        L.oracle_dequant64.argtypes = [i32, p, p, i64, i64, i64, i64, p]
        L.oracle_dequant64.restype = ctypes.c_int
        L.oracle_gemm.argtypes = [i32, p, p, i64, i64, p, i64, p, i64, p, p, i32]
        L.oracle_gemm.restype = ctypes.c_int
        L.oracle_last_threads.argtypes, L.oracle_last_threads.restype = [], i32
        L.oracle_swiglu.argtypes, L.oracle_swiglu.restype = [p, p, i64, p], None
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def fp16(bits: int) -> float:
    return lib().oracle_fp16(bits)


def e4m3(bits: int) -> float:
    return lib().oracle_e4m3(bits)


def e2m1(code: int) -> float:
    return lib().oracle_e2m1(code)


def bf16(bits: int) -> float:
    return lib().oracle_bf16(bits)


def row_bytes(wtype: int, k: int) -> int:
    return lib().oracle_row_bytes(wtype, k)


def dequant(wtype: int, data: np.ndarray, scales, m: int, k: int, r0: int = 0, nr=None) -> np.ndarray:
    """fp32 [nr, k] dequantized rows r0 .. r0+nr-1."""
    nr = m - r0 if nr is None else nr
    data = np.ascontiguousarray(data, dtype=np.uint8)
    scales = None if scales is None else np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty((nr, k), dtype=np.float32)
    rc = lib().oracle_dequant(wtype, _ptr(data), _ptr(scales), m, k, r0, nr, _ptr(out))
    if rc:
        raise ValueError("oracle_dequant: bad arguments")
    return out


def dequant64(wtype: int, data: np.ndarray, scales, m: int, k: int, r0: int = 0, nr=None) -> np.ndarray:
    """fp64 [nr, k]: the exact weights of rows r0 .. r0+nr-1 (dequant() rounds these
    once to fp32)."""
    nr = m - r0 if nr is None else nr
    data = np.ascontiguousarray(data, dtype=np.uint8)
    scales = None if scales is None else np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty((nr, k), dtype=np.float64)
    rc = lib().oracle_dequant64(wtype, _ptr(data), _ptr(scales), m, k, r0, nr, _ptr(out))
    if rc:
        raise ValueError("oracle_dequant64: bad arguments")
    return out


def gemm(wtype: int, data: np.ndarray, scales, m: int, k: int, x: np.ndarray,
         rows=None, nthreads: int = 0):
    """(y, a): y[t, i] = sum_k w[rows[i], k] x[t, k] in fp64, a = sum |w||x|.

    x is an fp16 array [n, k]; rows None means every row.
    """
    data = np.ascontiguousarray(data, dtype=np.uint8)
    scales = None if scales is None else np.ascontiguousarray(scales, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float16)
    if x.ndim == 1:
        x = x[None, :]
    n = x.shape[0]
    if x.shape[1] != k:
        raise ValueError("x has the wrong width")
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = m if r is None else r.shape[0]
    y = np.empty((n, nrows), dtype=np.float64)
    a = np.empty((n, nrows), dtype=np.float64)
    rc = lib().oracle_gemm(wtype, _ptr(data), _ptr(scales), m, k, _ptr(x.view(np.uint16)), n,
                           _ptr(r), nrows, _ptr(y), _ptr(a), nthreads)
    if rc:
        raise ValueError("oracle_gemm: bad arguments")
    return y, a


def last_threads() -> int:
    return lib().oracle_last_threads()


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    out = np.empty_like(g)
    lib().oracle_swiglu(_ptr(g), _ptr(u), g.size, _ptr(out))
    return out
