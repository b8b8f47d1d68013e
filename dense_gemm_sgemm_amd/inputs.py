"""Seeded synthetic inputs for the GEMM workloads.

This module holds generators and workload shapes only -- no GEMM arithmetic --
so that the GPU parity tests, the benchmark and the oracle's tests can all draw
the very same host arrays.

Recipe: ``numpy.random.default_rng(seed)``; seeds 1, 2 and 3 for A, B and C_in
(the SGEMM example on the page "异步拷贝与 Hopper/Blackwell 新特性" fills A and
B from seeds 1 and 2).  fp32 operands are uniform on [-1, 1) converted to
float32; fp16 operands are drawn in float64 and rounded to binary16 by numpy's
round-to-nearest-even cast.  The ragged fp16 workload draws normal(0, sd=0.5).
bfloat16 operands are the same draws converted to float32 and rounded to
bfloat16 (nearest, ties to even), kept as uint16 bit patterns since numpy has
no bfloat16 type.  All operands are packed row-major in their stored layout.
"""
from __future__ import annotations

import numpy as np

SEED_A, SEED_B, SEED_C = 1, 2, 3

# Workload shapes.  Names say what each one is.
WORKLOADS = {
    "sgemm_256": dict(kind="f32", M=256, N=256, K=256, alpha=1.0, betas=(0.0,), dist="uniform"),
    "sgemm_1024": dict(kind="f32", M=1024, N=1024, K=1024, alpha=1.0, betas=(0.0,), dist="uniform"),
    "sgemm_4096": dict(kind="f32", M=4096, N=4096, K=4096, alpha=1.0, betas=(0.0, 0.5),
                       dist="uniform"),
    "hgemm_nt_5376x5376x2048": dict(kind="f16_nt", M=5376, N=5376, K=2048, dist="uniform"),
    "hgemm_nt_5000x3001x1537": dict(kind="f16_nt", M=5000, N=3001, K=1537, dist="normal"),
    # a fused-QKV projection: 2048 tokens x 768 hidden -> 3 x 768 outputs
    "hgemm_nt_2048x2304x768": dict(kind="f16_nt", M=2048, N=2304, K=768, dist="uniform"),
    # a decode step: one token's hidden state (1 x 4096) times a 4096 -> 16384
    # projection stored as B[16384][4096]
    "hgemv_nt_1x16384x4096": dict(kind="f16_nt", M=1, N=16384, K=4096, dist="uniform"),
    # a single 128 x 128 output tile over a long K
    "hgemm_nt_128x128x16384": dict(kind="f16_nt", M=128, N=128, K=16384, dist="uniform"),
}


def uniform(shape, seed: int, dtype=np.float32) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.uniform(-1.0, 1.0, size=shape).astype(dtype)


def normal(shape, seed: int, sd: float = 0.5, dtype=np.float16) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, sd, size=shape).astype(dtype)


def small_ints(shape, seed: int, lo: int, hi: int, dtype) -> np.ndarray:
    """Integers drawn uniformly from [lo, hi] (inclusive), stored as ``dtype``."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape).astype(dtype)


def sgemm_operands(M: int, N: int, K: int, with_c: bool = False, dist: str = "uniform"):
    """A[M,K], B[K,N] (and C_in[M,N]) float32, row-major."""
    gen = uniform if dist == "uniform" else (lambda s, seed: normal(s, seed, dtype=np.float32))
    A = gen((M, K), SEED_A)
    B = gen((K, N), SEED_B)
    C = gen((M, N), SEED_C) if with_c else None
    return A, B, C


def hgemm_nt_operands(M: int, N: int, K: int, dist: str = "uniform"):
    """A[M,K] and B[N,K] binary16, row-major (C = A * B^T)."""
    if dist == "uniform":
        return uniform((M, K), SEED_A, np.float16), uniform((N, K), SEED_B, np.float16)
    return normal((M, K), SEED_A), normal((N, K), SEED_B)


def bf16_bits(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float64 draws: converted to float32,
    then rounded to bfloat16 on the float32 bits (nearest, ties to even).  The
    draws are finite."""
    bits = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    bits = bits + 0x7FFF + ((bits >> 16) & 1)
    return (bits >> 16).astype(np.uint16)


def operands16(shape_a, shape_b, fmt: str = "f16", dist: str = "normal"):
    """A and B of the given stored shapes, binary16 (float16 arrays) or
    bfloat16 (uint16 bit patterns), from seeds SEED_A and SEED_B."""
    if dist == "uniform":
        a = np.random.default_rng(SEED_A).uniform(-1.0, 1.0, size=shape_a)
        b = np.random.default_rng(SEED_B).uniform(-1.0, 1.0, size=shape_b)
    else:
        a = np.random.default_rng(SEED_A).normal(0.0, 0.5, size=shape_a)
        b = np.random.default_rng(SEED_B).normal(0.0, 0.5, size=shape_b)
    if fmt == "f16":
        return a.astype(np.float16), b.astype(np.float16)
    return bf16_bits(a), bf16_bits(b)


def workload_operands(name: str):
    w = WORKLOADS[name]
    if w["kind"] == "f32":
        return sgemm_operands(w["M"], w["N"], w["K"], with_c=any(b != 0 for b in w["betas"]),
                              dist=w["dist"])
    return hgemm_nt_operands(w["M"], w["N"], w["K"], dist=w["dist"])
