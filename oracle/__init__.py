"""CPU oracle for the tiled GEMM C = A x B -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``tiled_software_pipelined_amd``) and neither imports the other.

The arithmetic lives in ``tgemm_oracle.c`` (plain C, fp64 / int64
accumulation, OpenMP over rows).  This module only builds that file with gcc,
loads it with ctypes and marshals numpy arrays.  What is computed is the
definition of the product in "4.1 CUDA GEMM算子性能优化" (CUDA GEMM operator
optimisation), section 1.1, with the row-major indexing of its naive kernel
(section 3.1).

Pinned by ``tests/test_oracle_pins.py`` against closed forms (identity,
permutation, all-ones, rank-1, Sylvester-Hadamard, int8 extremes) and against
exact rational brute force on tiny shapes; the fp32 fused-multiply-add chain
variant is pinned against an exact rational emulation of single-precision
fma.  Every function here is pinned; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tgemm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def compile_source(src: str, out: str) -> str:
    """Compile one C source of the oracle into a shared library (gcc, OpenMP)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-fPIC", "-shared", "-Wall", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ``tgemm_oracle.c`` into ``liboracle.so`` next to it (gcc)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    return compile_source(_SRC, _LIB_PATH)


def bind(path: str):
    """Open a compiled oracle library at ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    for name in ("oracle_gemm_f32", "oracle_gemm_bf16"):
        f = getattr(lib, name)
        f.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, vp, i64]
        f.restype = ctypes.c_int
    lib.oracle_gemm_i8.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64]
    lib.oracle_gemm_i8.restype = ctypes.c_int
    lib.oracle_gemm_f32_fma_chain.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64]
    lib.oracle_gemm_f32_fma_chain.restype = ctypes.c_int
    for name in ("oracle_gemm_f32_sampled", "oracle_gemm_bf16_sampled"):
        f = getattr(lib, name)
        f.argtypes = [i64, i64, i64, vp, i64, vp, i64, i64, vp, vp, vp, vp]
        f.restype = ctypes.c_int
    lib.oracle_gemm_i8_sampled.argtypes = [i64, i64, i64, vp, i64, vp, i64, i64, vp, vp, vp]
    lib.oracle_gemm_i8_sampled.restype = ctypes.c_int
    lib.oracle_gemm_f32_fma_chain_sampled.argtypes = [i64, i64, i64, vp, i64, vp, i64,
                                                      i64, vp, vp, vp]
    lib.oracle_gemm_f32_fma_chain_sampled.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = bind(_LIB_PATH)
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


_DT = {"f32": np.float32, "bf16": np.uint16, "i8": np.int8}


def _operand(x, dtype_name):
    """Return (array, leading dim).  Rows may be padded (row stride > cols)."""
    want = _DT[dtype_name]
    x = np.asarray(x)
    if x.dtype != want:
        raise TypeError("oracle %s operand must be %s, got %s" % (dtype_name, want, x.dtype))
    if x.ndim != 2:
        raise ValueError("operand must be 2-D")
    if x.strides[1] != x.itemsize or x.strides[0] % x.itemsize:
        x = np.ascontiguousarray(x)
    ld = x.strides[0] // x.itemsize if x.shape[0] > 1 else max(x.shape[1], 1)
    return x, ld


def _ptr(x):
    return x.ctypes.data_as(ctypes.c_void_p)


def gemm(A, B, dtype: str):
    """Full reference product.

    ``dtype`` is "f32" (float32 operands), "bf16" (raw bf16 bit patterns as
    uint16) or "i8" (int8).  Returns ``(C, S)``: fp64 C and fp64
    S = sum_k |a_ik b_kj| for the float types; exact int64 C and ``None`` for
    int8.  A may be a row-padded view (its row stride is used as lda).
    """
    lib = _load()
    A, lda = _operand(A, dtype)
    B, ldb = _operand(B, dtype)
    M, K = A.shape
    K2, N = B.shape
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    if dtype == "i8":
        C = np.zeros((M, N), dtype=np.int64)
        rc = lib.oracle_gemm_i8(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), max(N, 1))
        S = None
    else:
        C = np.zeros((M, N), dtype=np.float64)
        S = np.zeros((M, N), dtype=np.float64)
        f = lib.oracle_gemm_f32 if dtype == "f32" else lib.oracle_gemm_bf16
        rc = f(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), _ptr(S), max(N, 1))
    if rc != 0:
        raise ValueError("oracle rejected the sizes")
    return C, S


def gemm_f32_fma_chain(A, B):
    """fp32 product with one single-precision fma chain per output, k increasing."""
    lib = _load()
    A, lda = _operand(A, "f32")
    B, ldb = _operand(B, "f32")
    M, K = A.shape
    N = B.shape[1]
    if B.shape[0] != K:
        raise ValueError("inner dimensions differ")
    C = np.zeros((M, N), dtype=np.float32)
    rc = lib.oracle_gemm_f32_fma_chain(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), max(N, 1))
    if rc != 0:
        raise ValueError("oracle rejected the sizes")
    return C


def gemm_sampled(A, B, rows, cols, dtype: str, fma_chain: bool = False):
    """Reference values at positions (rows[p], cols[p]) only.

    Returns ``(C, S)`` as 1-D arrays (``S`` is None for int8 and for the fp32
    fma chain, whose C is float32).
    """
    lib = _load()
    A, lda = _operand(A, dtype)
    B, ldb = _operand(B, dtype)
    M, K = A.shape
    N = B.shape[1]
    if B.shape[0] != K:
        raise ValueError("inner dimensions differ")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    P = rows.shape[0]
    if cols.shape[0] != P:
        raise ValueError("rows and cols differ in length")
    if fma_chain:
        if dtype != "f32":
            raise ValueError("the fma chain reference is fp32 only")
        C = np.zeros(P, dtype=np.float32)
        rc = lib.oracle_gemm_f32_fma_chain_sampled(M, N, K, _ptr(A), lda, _ptr(B), ldb, P,
                                                   _ptr(rows), _ptr(cols), _ptr(C))
        S = None
    elif dtype == "i8":
        C = np.zeros(P, dtype=np.int64)
        rc = lib.oracle_gemm_i8_sampled(M, N, K, _ptr(A), lda, _ptr(B), ldb, P,
                                        _ptr(rows), _ptr(cols), _ptr(C))
        S = None
    else:
        C = np.zeros(P, dtype=np.float64)
        S = np.zeros(P, dtype=np.float64)
        f = lib.oracle_gemm_f32_sampled if dtype == "f32" else lib.oracle_gemm_bf16_sampled
        rc = f(M, N, K, _ptr(A), lda, _ptr(B), ldb, P, _ptr(rows), _ptr(cols), _ptr(C), _ptr(S))
    if rc != 0:
        raise ValueError("oracle rejected the sizes or positions")
    return C, S
