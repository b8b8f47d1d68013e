"""A seeded random sweep across the paths: shapes drawn so that every kernel
family is reached (streaming, register-staged full and wide tiles, edge,
split-K through the explicit calls, matrix-vector, the ragged forms of the
full and streaming tiles), with padded leading
dimensions and, for fp32, random alpha and beta.  Products up to 2^27 multiply-adds are compared element by element
with the oracle, larger ones on sampled outputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from dense_gemm_sgemm_amd import inputs
from tolerance import f16_check, f32_check, f32_tolerance

torch = pytest.importorskip("torch")
import dense_gemm_sgemm_amd as dg  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def draw(seed):
    rng = np.random.default_rng(seed)
    kind = "f32" if seed % 2 == 0 else "f16"
    family = rng.integers(0, 5) if seed < 48 else 5
    if family == 0:       # small and ragged
        M, N, K = (int(x) for x in rng.integers(1, 300, 3))
    elif family == 1:     # whole tiles
        M, N, K = (int(x) for x in 64 * rng.integers(1, 40, 3))
    elif family == 2:     # large and ragged (register-staged wide fp16 tiles, fp32 edge)
        M, N, K = (int(x) for x in rng.integers(900, 2600, 3))
    elif family == 3:     # few tiles, long K (split-K)
        M, N, K = int(rng.integers(1, 400)), int(rng.integers(1, 400)), int(rng.integers(2048, 9000))
    elif family == 4:     # thin (matrix-vector for fp16)
        M, N, K = int(rng.integers(1, 9)), int(rng.integers(100, 5000)), int(rng.integers(1, 3000))
        if rng.integers(0, 2):
            M, N = N, M
    else:                 # large and ragged, rows at 16-byte addresses (the ragged full tiles)
        M, N = (int(x) for x in rng.integers(1000, 5000, 2))
        K = 8 * int(rng.integers(9, 400))
        if kind == "f32":
            N -= N % 4    # fp32 B and C rows at 16-byte addresses too
        pad = int(rng.choice([0, 8]))
        alpha, beta = [(1.0, 0.0), (0.5, 1.0), (-1.5, 0.25)][int(rng.integers(0, 3))]
        return kind, M, N, K, pad, alpha, beta, False
    pad = int(rng.choice([0, 0, 1, 4, 8]))
    alpha, beta = [(1.0, 0.0), (0.5, 1.0), (-1.5, 0.25)][int(rng.integers(0, 3))]
    return kind, M, N, K, pad, alpha, beta, int(family) == 3


SEEDS = list(range(64))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_sweep(seed):
    kind, M, N, K, pad, alpha, beta, split = draw(seed)
    print("\n[sweep] seed %d %s %dx%dx%d pad %d alpha %g beta %g" % (seed, kind, M, N, K, pad, alpha, beta),
          flush=True)
    sys.stdout.flush()
    small = M * N * K <= (1 << 27)
    rng = np.random.default_rng(1000 + seed)
    if small:
        rows = cols = None
    else:
        # the first and last rows and columns whole (the shifted edge tiles of
        # the ragged forms end there), and random points
        rows = np.concatenate([np.zeros(N, np.int64), np.full(N, M - 1), np.arange(M), np.arange(M),
                               rng.integers(0, M, 4000)])
        cols = np.concatenate([np.arange(N), np.arange(N), np.zeros(M, np.int64), np.full(M, N - 1),
                               rng.integers(0, N, 4000)])
    if kind == "f32":
        A, B, C = inputs.sgemm_operands(M, N, K, with_c=True)
        bA = torch.zeros(M, K + pad, device=DEV); bA[:, :K] = torch.from_numpy(A).to(DEV)
        bB = torch.zeros(K, N + pad, device=DEV); bB[:, :N] = torch.from_numpy(B).to(DEV)
        bC = torch.full((M, N + pad), 3.0, device=DEV); bC[:, :N] = torch.from_numpy(C).to(DEV)
        path = dg.f32_path(bA[:, :K], bB[:, :N], bC[:, :N], alpha, beta)
        if split:
            path += " (split-K call)"
            dg.gemm_f32_splitk(bA[:, :K], bB[:, :N], bC[:, :N], alpha, beta)
        else:
            dg.gemm_f32(bA[:, :K], bB[:, :N], bC[:, :N], alpha, beta)
        torch.cuda.synchronize()
        got = bC.cpu().numpy()
        assert np.all(got[:, N:] == 3.0)
        tol = f32_tolerance(K, 1.0, 1.0, alpha, beta, 1.0)
        if small:
            f32_check(got[:, :N], oracle.gemm_f32(A, B, alpha, beta, C), tol)
        else:
            f32_check(got[:, :N][rows, cols], oracle.gemm_f32_points(A, B, rows, cols, alpha, beta, C), tol)
    else:
        A, B = inputs.hgemm_nt_operands(M, N, K)
        bA = torch.zeros(M, K + pad, device=DEV, dtype=torch.float16); bA[:, :K] = torch.from_numpy(A).to(DEV)
        bB = torch.zeros(N, K + pad, device=DEV, dtype=torch.float16); bB[:, :K] = torch.from_numpy(B).to(DEV)
        bC = torch.full((M, N + pad), 3.0, device=DEV, dtype=torch.float16)
        path = dg.f16_nt_path(bA[:, :K], bB[:, :K], bC[:, :N])
        if split:
            path += " (split-K call)"
            dg.gemm_f16_nt_splitk(bA[:, :K], bB[:, :K], bC[:, :N])
        else:
            dg.gemm_f16_nt(bA[:, :K], bB[:, :K], bC[:, :N])
        torch.cuda.synchronize()
        got = bC.cpu().numpy()
        assert np.all(got[:, N:] == 3.0)
        absA = (A.view(np.uint16) & np.uint16(0x7FFF)).view(np.float16)
        absB = (B.view(np.uint16) & np.uint16(0x7FFF)).view(np.float16)
        if small:
            f16_check(got[:, :N], oracle.gemm_f16_nt_exact(A, B), oracle.gemm_f16_nt_exact(absA, absB))
        else:
            f16_check(got[:, :N][rows, cols], oracle.gemm_f16_nt_points(A, B, rows, cols),
                      oracle.gemm_f16_nt_points(absA, absB, rows, cols))
    print("[sweep] seed %d path %s ok" % (seed, path), flush=True)
