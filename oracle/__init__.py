"""CPU oracle for the dense GEMM path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports it and it
imports nothing from the GPU library: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64 accumulation, OpenMP over
rows); this module only builds it with gcc, loads it with ctypes and marshals
numpy arrays.  Definitions followed (see the header of ``oracle.c``):

* ``gemm_f32``: row-major ``C = alpha*A*B + beta*C`` -- the cp.async SGEMM
  example of the page "异步拷贝与 Hopper/Blackwell 新特性" and the naive loop
  of page 1 section 6.1.  ``beta == 0`` means C is not read.
* ``gemm_f16_nt``: ``C = A*B^T`` with A[M][K], B[N][K] binary16 -- section "0.
  Naive Implementation" of the page "从零开始的 AI Infra: 算子基础与GPU架构",
  summed in double and rounded once to half (nearest, ties to even).
* ``f16_epilogue`` / ``gemm_f16_nt_ex``: the fused write-back of page 1
  section 6.5.4, ``C = act(A*B^T + bias) + residual`` (act none, ReLU or
  SiLU), in double before the one rounding.
* ``bf16_*`` and the ``fmt="bf16"`` arguments: the same products on bfloat16
  operands (page 1 section 6.3.3 names bf16 beside fp16 as a matrix-unit
  input type), rounded once to bfloat16.  numpy has no bfloat16 dtype, so
  bfloat16 arrays are uint16 bit patterns here.
* ``gemm_ex_exact``: the products for the other operand layouts (A stored
  K x M, B stored K x N), by transposing the stored operands first.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_i = ctypes.c_int
_l = ctypes.c_long
_d = ctypes.c_double
_p = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (no fast-math)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-Wall", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _configure(lib):
    """Declare the C signatures on a loaded copy of the oracle library."""
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = _d
    lib.oracle_half_from_double.argtypes = [_d]
    lib.oracle_half_from_double.restype = ctypes.c_uint16
    lib.oracle_half_round_array.argtypes = [_l, _p, _p]
    lib.oracle_half_decode_array.argtypes = [_l, _p, _p]
    lib.oracle_gemm_f32.argtypes = [_i, _i, _i, _d, _p, _l, _p, _l, _d, _p, _l, _p, _l]
    lib.oracle_gemm_f32_points.argtypes = [_i, _d, _p, _l, _p, _l, _d, _p, _l, _l, _p, _p, _p]
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = _d
    lib.oracle_bf16_from_double.argtypes = [_d]
    lib.oracle_bf16_from_double.restype = ctypes.c_uint16
    lib.oracle_bf16_round_array.argtypes = [_l, _p, _p]
    lib.oracle_bf16_decode_array.argtypes = [_l, _p, _p]
    lib.oracle_gemm_16_nt.argtypes = [_i, _i, _i, _i, _p, _l, _p, _l, _p, _l]
    lib.oracle_gemm_16_nt_points.argtypes = [_i, _i, _p, _l, _p, _l, _l, _p, _p, _p]
    lib.oracle_epilogue16.argtypes = [_i, _l, _p, _p, _p, _p, _i, _p, _l, _p]
    lib.oracle_max_threads.restype = _i
    lib.oracle_set_threads.argtypes = [_i]
    for fn in (lib.oracle_half_round_array, lib.oracle_half_decode_array,
               lib.oracle_bf16_round_array, lib.oracle_bf16_decode_array, lib.oracle_gemm_f32,
               lib.oracle_gemm_f32_points, lib.oracle_gemm_16_nt, lib.oracle_gemm_16_nt_points,
               lib.oracle_epilogue16, lib.oracle_set_threads):
        fn.restype = None
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            build()
        lib = _configure(ctypes.CDLL(_LIB))
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _rows(a: np.ndarray, dtype) -> tuple[np.ndarray, int]:
    """A 2-D array whose rows may be strided but whose elements are packed."""
    if a.dtype != dtype or a.ndim != 2:
        raise TypeError("expected a 2-D %s array" % np.dtype(dtype).name)
    if a.strides[1] != a.itemsize or a.strides[0] % a.itemsize:
        a = np.ascontiguousarray(a)
    ld = a.strides[0] // a.itemsize if a.shape[0] > 1 else max(1, a.shape[1])
    return a, ld


def max_threads() -> int:
    return _load().oracle_max_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def half_from_double(x) -> np.ndarray:
    """Round float64 values to binary16 (nearest, ties to even); returns float16."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_half_round_array(x.size, _ptr(x), _ptr(out))
    return out.view(np.float16)


def half_to_double(h) -> np.ndarray:
    h = np.ascontiguousarray(np.asarray(h, dtype=np.float16)).view(np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    _load().oracle_half_decode_array(h.size, _ptr(h), _ptr(out))
    return out


def bf16_from_double(x) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_bf16_round_array(x.size, _ptr(x), _ptr(out))
    return out


def bf16_to_double(b) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_bf16_decode_array(b.size, _ptr(b), _ptr(out))
    return out


# 16-bit storage formats: numpy dtype of the arrays, code in oracle.c, rounding.
_FMT = {"f16": (np.float16, 0), "bf16": (np.uint16, 1)}


def round16(x, fmt: str) -> np.ndarray:
    """Round float64 values to the format (float16 array, or uint16 bfloat16 bits)."""
    return half_from_double(x) if fmt == "f16" else bf16_from_double(x)


def decode16(a, fmt: str) -> np.ndarray:
    return half_to_double(a) if fmt == "f16" else bf16_to_double(a)


def gemm_f32(A: np.ndarray, B: np.ndarray, alpha: float = 1.0, beta: float = 0.0,
             C: np.ndarray | None = None) -> np.ndarray:
    """fp64 value of ``alpha*A@B + beta*C`` for float32 A[M,K], B[K,N], C[M,N]."""
    A, lda = _rows(A, np.float32)
    B, ldb = _rows(B, np.float32)
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    alpha = float(np.float32(alpha))
    beta = float(np.float32(beta))
    if beta != 0.0:
        if C is None or C.shape != (M, N):
            raise ValueError("beta != 0 needs C of shape (M, N)")
        C, ldc = _rows(C, np.float32)
        cptr = _ptr(C)
    else:
        ldc, cptr = 1, None
    out = np.empty((M, N), dtype=np.float64)
    _load().oracle_gemm_f32(M, N, K, alpha, _ptr(A), lda, _ptr(B), ldb, beta, cptr, ldc,
                            _ptr(out), max(N, 1))
    return out


def gemm_f32_points(A, B, rows, cols, alpha: float = 1.0, beta: float = 0.0, C=None) -> np.ndarray:
    """The same value as :func:`gemm_f32`, at the outputs (rows[t], cols[t]) only."""
    A, lda = _rows(A, np.float32)
    B, ldb = _rows(B, np.float32)
    K = A.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    alpha = float(np.float32(alpha))
    beta = float(np.float32(beta))
    if beta != 0.0:
        C, ldc = _rows(C, np.float32)
        cptr = _ptr(C)
    else:
        ldc, cptr = 1, None
    out = np.empty(rows.shape, dtype=np.float64)
    _load().oracle_gemm_f32_points(K, alpha, _ptr(A), lda, _ptr(B), ldb, beta, cptr, ldc,
                                   rows.size, _ptr(rows), _ptr(cols), _ptr(out))
    return out


def gemm_16_nt_exact(A: np.ndarray, B: np.ndarray, fmt: str = "f16") -> np.ndarray:
    """fp64 sum ``A @ B.T`` for 16-bit A[M,K], B[N,K] (binary16 as float16 arrays,
    bfloat16 as uint16 bit patterns), before output rounding."""
    dtype, code = _FMT[fmt]
    A, lda = _rows(A, dtype)
    B, ldb = _rows(B, dtype)
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    out = np.empty((M, N), dtype=np.float64)
    _load().oracle_gemm_16_nt(code, M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(out), max(N, 1))
    return out


def gemm_16_nt_points(A, B, rows, cols, fmt: str = "f16") -> np.ndarray:
    """fp64 sums of :func:`gemm_16_nt_exact` at the outputs (rows[t], cols[t])."""
    dtype, code = _FMT[fmt]
    A, lda = _rows(A, dtype)
    B, ldb = _rows(B, dtype)
    K = A.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    out = np.empty(rows.shape, dtype=np.float64)
    _load().oracle_gemm_16_nt_points(code, K, _ptr(A), lda, _ptr(B), ldb, rows.size,
                                     _ptr(rows), _ptr(cols), _ptr(out))
    return out


def gemm_f16_nt_exact(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """fp64 sum ``A @ B.T`` for binary16 A[M,K], B[N,K], before output rounding."""
    return gemm_16_nt_exact(A, B, "f16")


def gemm_f16_nt(A: np.ndarray, B: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Returns (fp64 sum, that sum rounded to binary16) for ``C = A @ B.T``."""
    ref = gemm_f16_nt_exact(A, B)
    return ref, half_from_double(ref)


def gemm_f16_nt_points(A, B, rows, cols) -> np.ndarray:
    """fp64 sums of :func:`gemm_f16_nt_exact` at the outputs (rows[t], cols[t])."""
    return gemm_16_nt_points(A, B, rows, cols, "f16")


def gemm_bf16_nt(A: np.ndarray, B: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Returns (fp64 sum, that sum rounded to bfloat16 bits) for ``C = A @ B.T``
    on bfloat16 bit patterns A[M,K], B[N,K] (uint16)."""
    ref = gemm_16_nt_exact(A, B, "bf16")
    return ref, bf16_from_double(ref)


ACTS = {"none": 0, "relu": 1, "silu": 2}


def epilogue16(acc, rows, cols, bias=None, act="none", residual=None, fmt: str = "f16"):
    """fp64 ``act(acc + bias[col]) + residual[row, col]`` at the outputs
    (rows[t], cols[t]), ``acc[t]`` being the product's sum there; bias and
    residual in the 16-bit format ``fmt``."""
    dtype, code = _FMT[fmt]
    acc = np.ascontiguousarray(acc, dtype=np.float64).ravel()
    rows = np.ascontiguousarray(rows, dtype=np.int32).ravel()
    cols = np.ascontiguousarray(cols, dtype=np.int32).ravel()
    if not (acc.size == rows.size == cols.size):
        raise ValueError("acc, rows and cols differ in length")
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=dtype).ravel()
    ldres = 0
    if residual is not None:
        residual, ldres = _rows(residual, dtype)
    out = np.empty(acc.shape, dtype=np.float64)
    _load().oracle_epilogue16(code, acc.size, _ptr(acc), _ptr(rows), _ptr(cols),
                              None if bias is None else _ptr(bias), ACTS[act],
                              None if residual is None else _ptr(residual), ldres, _ptr(out))
    return out


def f16_epilogue(acc, rows, cols, bias=None, act="none", residual=None) -> np.ndarray:
    """:func:`epilogue16` on binary16 bias and residual."""
    return epilogue16(acc, rows, cols, bias, act, residual, "f16")


def gemm_16_nt_ex_exact(A, B, bias=None, act="none", residual=None, fmt: str = "f16"):
    """fp64 ``act(A @ B.T + bias) + residual`` (before the output rounding)."""
    acc = gemm_16_nt_exact(A, B, fmt)
    M, N = acc.shape
    rr, cc = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    return epilogue16(acc, rr, cc, bias, act, residual, fmt).reshape(M, N)


def gemm_f16_nt_ex_exact(A, B, bias=None, act="none", residual=None) -> np.ndarray:
    return gemm_16_nt_ex_exact(A, B, bias, act, residual, "f16")


def gemm_f16_nt_ex(A, B, bias=None, act="none", residual=None):
    """(fp64 value, that value rounded to binary16) of the fused product."""
    ref = gemm_f16_nt_ex_exact(A, B, bias, act, residual)
    return ref, half_from_double(ref)


def nt_operands(A_stored, B_stored, op_a: str, op_b: str):
    """The A[M,K] and B[N,K] of ``C = op(A) @ op(B)``: op "n" keeps A as M x K
    and B as K x N, op "t" reads A stored K x M and B stored N x K."""
    A = A_stored if op_a == "n" else np.ascontiguousarray(A_stored.T)
    B = B_stored if op_b == "t" else np.ascontiguousarray(B_stored.T)
    return A, B


def gemm_ex_exact(A_stored, B_stored, op_a: str = "n", op_b: str = "t", bias=None, act="none",
                  residual=None, fmt: str = "f16") -> np.ndarray:
    """fp64 ``act(op(A) @ op(B) + bias) + residual`` for 16-bit operands in any
    of the four layouts, before the output rounding."""
    A, B = nt_operands(A_stored, B_stored, op_a, op_b)
    return gemm_16_nt_ex_exact(A, B, bias, act, residual, fmt)
