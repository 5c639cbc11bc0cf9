"""Plain CPU oracle for Y[M,N] = X[M,K] . W[N,K]^T with bf16 inputs.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library never
loads it, and this package imports nothing from the HIP library.

The arithmetic lives in ``oracle.c`` (plain C, fp64): each bf16 is widened to
double exactly, every output is the ascending-k double sum of exact products,
and the final value is rounded once to f32 or once to bf16 (IEEE
round-to-nearest-even).  What it follows: the numerical contract of the blog
series "On descend d'un cran" -- bf16 weights and activations with f32
accumulation (post 0, section "Ce qu'il y aura dans le depot"), results that
differ between correct engines only by summation order ("#002 le meme
compilateur sur un GPU", section "Le contrat numerique"), and IEEE-rounded
arithmetic with a single rounding where the reference rounds ("#004 the same
compiler on Apple's chips", opening sections).

bf16 tensors cross this interface as numpy ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-shared", "-fPIC", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
        lib.oracle_f64_to_f32.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_f32.restype = ctypes.c_float
        lib.oracle_matmul.argtypes = [_p, _p, _i64, _i64, _i64, _p, ctypes.c_int]
        lib.oracle_matmul.restype = None
        lib.oracle_matmul_rows.argtypes = [_p, _p, _i64, _p, _i64, _i64, _p, ctypes.c_int]
        lib.oracle_matmul_rows.restype = None
        lib.oracle_round_f32.argtypes = [_p, _p, _i64]
        lib.oracle_round_f32.restype = None
        lib.oracle_round_bf16.argtypes = [_p, _p, _i64]
        lib.oracle_round_bf16.restype = None
        lib.oracle_round_f32_to_bf16.argtypes = [_p, _p, _i64, ctypes.c_int]
        lib.oracle_round_f32_to_bf16.restype = None
        lib.oracle_rmsnorm.argtypes = [_p, _p, _i64, _i64, ctypes.c_double, _p]
        lib.oracle_rmsnorm.restype = None
        lib.oracle_rmsnorm_matmul.argtypes = [_p, _p, _p, _i64, _i64, _i64, ctypes.c_double, ctypes.c_int, _p,
                                              ctypes.c_int]
        lib.oracle_rmsnorm_matmul.restype = None
        lib.oracle_swiglu.argtypes = [_p, _i64, _i64, _p]
        lib.oracle_swiglu.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def _u16(a: np.ndarray, name: str) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name} must hold bf16 bit patterns as uint16, got {a.dtype}")
    return a


def matmul(X: np.ndarray, W: np.ndarray, threads: int = 0) -> np.ndarray:
    """Exact-to-fp64 Y[M,N] = X[M,K] . W[N,K]^T; X, W are uint16 bf16 bits."""
    X = _u16(X, "X")
    W = _u16(W, "W")
    M, K = X.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError(f"K mismatch: X has {K}, W has {K2}")
    Y = np.empty((M, N), dtype=np.float64)
    if M * N:
        _load().oracle_matmul(X.ctypes.data, W.ctypes.data, M, N, K, Y.ctypes.data, threads)
    return Y


def matmul_rows(X: np.ndarray, rows, W: np.ndarray, threads: int = 0) -> np.ndarray:
    """Rows ``rows`` of the fp64 product (X is the full matrix)."""
    X = _u16(X, "X")
    W = _u16(W, "W")
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    M, K = X.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError("K mismatch")
    if rows.size and (rows.min() < 0 or rows.max() >= M):
        raise IndexError("row index out of range")
    Y = np.empty((rows.size, N), dtype=np.float64)
    if rows.size * N:
        _load().oracle_matmul_rows(X.ctypes.data, rows.ctypes.data, rows.size,
                                   W.ctypes.data, N, K, Y.ctypes.data, threads)
    return Y


def swiglu(Y: np.ndarray) -> np.ndarray:
    """H[m, j] = silu(Y[m, j]) * Y[m, N/2 + j] in fp64 for an fp64 gate_up
    product Y [M, N] (gate columns first, then up), N even; see oracle.c."""
    Y = np.ascontiguousarray(Y, dtype=np.float64)
    if Y.ndim != 2 or Y.shape[1] % 2:
        raise ValueError("swiglu: Y must be [M, N] with N even")
    M, N = Y.shape
    H = np.empty((M, N // 2), dtype=np.float64)
    if H.size:
        _load().oracle_swiglu(Y.ctypes.data, M, N, H.ctypes.data)
    return H


def rmsnorm(X: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """fp64 RMS-normalised rows of X (bf16 bits [M, K]) with f32 gamma [K]; see oracle.c."""
    X = _u16(X, "X")
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    M, K = X.shape
    if g.shape != (K,):
        raise ValueError("gamma must have K values")
    out = np.empty((M, K), dtype=np.float64)
    if out.size:
        _load().oracle_rmsnorm(X.ctypes.data, g.ctypes.data, M, K, float(eps), out.ctypes.data)
    return out


def rmsnorm_matmul(X: np.ndarray, gamma: np.ndarray, W: np.ndarray, eps: float, absolute: bool = False,
                   threads: int = 0) -> np.ndarray:
    """fp64 projection of the RMS-normalised rows (or, with absolute, the sums of
    the terms' magnitudes); see oracle.c."""
    X = _u16(X, "X")
    W = _u16(W, "W")
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    M, K = X.shape
    N, K2 = W.shape
    if K != K2 or g.shape != (K,):
        raise ValueError("shape mismatch")
    out = np.empty((M, N), dtype=np.float64)
    if out.size:
        _load().oracle_rmsnorm_matmul(X.ctypes.data, g.ctypes.data, W.ctypes.data, M, N, K, float(eps),
                                      1 if absolute else 0, out.ctypes.data, threads)
    return out


PANEL_ROWS = 128
PANEL_COLS = 64


def pack_panels(W: np.ndarray) -> np.ndarray:
    """W [N, K] (row-major) in the library's packed weight layout, as an array of
    shape (N/128, K/64, 128, 64) whose C order is the packed memory order:
    element [p, b, r, q] is W[128 p + r, 64 b + q] -- 128-row panels, each as
    K/64 consecutive blocks of 128 rows x 64 values, each block row-major.
    This layout is the library's own (declared with proj_pack_weights); the
    pages behind it pack weights so that the kernel reads them in the order it
    consumes them ("#001 un compilateur pour moteur de LLM", section "Lire le
    meme emetteur rempli deux fois": 16-column blocks a fixed distance apart)
    and leave the GPU benefit to be measured kernel by kernel ("#002 le meme
    compilateur sur un GPU", section "Les autres cartes").  Written as one
    block copy per (panel, block); values are moved, never changed."""
    W = np.asarray(W)
    N, K = W.shape
    if N % PANEL_ROWS or K % PANEL_COLS:
        raise ValueError(f"packed layout needs N % 128 == 0 and K % 64 == 0, got {N}x{K}")
    out = np.empty((N // PANEL_ROWS, K // PANEL_COLS, PANEL_ROWS, PANEL_COLS), dtype=W.dtype)
    for p in range(N // PANEL_ROWS):
        for b in range(K // PANEL_COLS):
            out[p, b] = W[p * PANEL_ROWS:(p + 1) * PANEL_ROWS, b * PANEL_COLS:(b + 1) * PANEL_COLS]
    return out


def round_f32(Y: np.ndarray) -> np.ndarray:
    """Round fp64 results once to f32 (IEEE RNE)."""
    Y = np.ascontiguousarray(Y, dtype=np.float64)
    out = np.empty(Y.shape, dtype=np.float32)
    if Y.size:
        _load().oracle_round_f32(Y.ctypes.data, out.ctypes.data, Y.size)
    return out


def round_bf16(Y: np.ndarray) -> np.ndarray:
    """Round fp64 results once to bf16 (IEEE RNE); returns uint16 bit patterns."""
    Y = np.ascontiguousarray(Y, dtype=np.float64)
    out = np.empty(Y.shape, dtype=np.uint16)
    if Y.size:
        _load().oracle_round_bf16(Y.ctypes.data, out.ctypes.data, Y.size)
    return out


def round_f32_to_bf16(F: np.ndarray, threads: int = 0) -> np.ndarray:
    """Round f32 values once to bf16 (IEEE RNE); returns uint16 bit patterns."""
    F = np.ascontiguousarray(F, dtype=np.float32)
    out = np.empty(F.shape, dtype=np.uint16)
    if F.size:
        _load().oracle_round_f32_to_bf16(F.ctypes.data, out.ctypes.data, F.size, threads)
    return out


def f64_to_bf16(x: float) -> int:
    return int(_load().oracle_f64_to_bf16(float(x)))


def bf16_to_f64(b: int) -> float:
    return float(_load().oracle_bf16_to_f64(int(b)))


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Widen an array of bf16 bit patterns to float64 (exact)."""
    a = np.asarray(a, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def max_threads() -> int:
    return int(_load().oracle_max_threads())
