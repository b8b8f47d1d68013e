"""HIP graph capture: the library's calls recorded with torch.cuda.graph and
replayed.  The library allocates nothing, so capture records only its
kernels; the calls that take a workspace (explicit split-K, gemm_ex's
transposed copies) get one allocated before capture (gemm_ex's in-place
layouts are given one too, and leave it untouched).  Each graph is replayed
several times, with the program's own eager work and synchronisations in
between, and every replay must equal the eager result bit for bit (the
kernels are deterministic and the path choice is the same)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from dense_gemm_sgemm_amd import inputs

torch = pytest.importorskip("torch")
import dense_gemm_sgemm_amd as dg  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    ("f32", (2048, 2048, 256), "f32_mfma"),
    ("f32", (1030, 1100, 1000), "f32_general"),
    ("f32_splitk", (512, 512, 16384), "f32_mfma"),
    ("f16", (512, 512, 512), "f16_mfma"),
    ("f16", (1000, 1030, 1100), "f16_staged"),
    ("f16_splitk", (128, 128, 16384), "f16_mfma"),
    ("ex_nn", (500, 301, 153), "f16_general"),
    # B stored [K][N] read in place: whole 128 x 192 tiles, and the ragged form
    ("ex_nn", (2048, 2304, 768), "f16_mfma"),
    ("ex_nn", (4100, 4200, 1024), "f16_mfma"),
]


def operands(kind, M, N, K):
    if kind.startswith("f32"):
        A, B, _ = inputs.sgemm_operands(M, N, K)
        return (torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV),
                torch.empty(M, N, device=DEV))
    A, B = inputs.hgemm_nt_operands(M, N, K)
    dB = torch.from_numpy(B).to(DEV)
    if kind == "ex_nn":
        dB = dB.t().contiguous()            # B stored K x N
    return (torch.from_numpy(A).to(DEV), dB,
            torch.empty(M, N, device=DEV, dtype=torch.float16))


def workspace(kind, A, B, C):
    """The workspace a call takes (allocated outside the capture), or None."""
    M, N = C.shape
    K = A.shape[1]
    if kind == "f32_splitk":
        n = dg.splitk_workspace_bytes("f32", M, N, K)
    elif kind == "f16_splitk":
        n = dg.splitk_workspace_bytes("f16", M, N, K)
    elif kind == "ex_nn":
        n = dg.ex_workspace_bytes(A, B, C, "n", "n")
    else:
        return None
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def call(kind, A, B, C, ws=None):
    if kind == "f32":
        dg.gemm_f32(A, B, C, 1.0, 0.0)
    elif kind == "f32_splitk":
        dg.gemm_f32_splitk(A, B, C, 1.0, 0.0, workspace=ws)
    elif kind == "f16_splitk":
        dg.gemm_f16_nt_splitk(A, B, C, workspace=ws)
    elif kind == "ex_nn":
        dg.gemm_ex(A, B, C, "n", "n", workspace=ws)
    else:
        dg.gemm_f16_nt(A, B, C)


def path(kind, A, B, C):
    if kind.startswith("f32"):
        return dg.f32_path(A, B, C)
    if kind == "ex_nn":
        return dg.ex_path(A, B, C, "n", "n")
    return dg.f16_nt_path(A, B, C)


@pytest.mark.parametrize("kind,shape,expect", CASES, ids=lambda x: str(x))
def test_graph_replays_equal_eager(kind, shape, expect):
    M, N, K = shape
    print("\n[graph case] %s %s %s" % (kind, shape, expect), flush=True)
    sys.stdout.flush()
    A, B, C = operands(kind, M, N, K)
    assert path(kind, A, B, C) == expect
    ws = workspace(kind, A, B, C)
    call(kind, A, B, C, ws)
    torch.cuda.synchronize()
    eager = C.clone()
    C.fill_(float("nan"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(kind, A, B, C, ws)
    torch.cuda.synchronize()
    A2, B2, C2 = operands(kind, M, N, K)
    ws2 = workspace(kind, A2, B2, C2)
    for _ in range(3):
        C.fill_(float("nan"))
        call(kind, A2, B2, C2, ws2)       # eager work on other buffers between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bits = torch.int32 if kind.startswith("f32") else torch.int16
        assert torch.equal(C.view(bits), eager.view(bits))
    assert torch.equal(C2.view(bits), eager.view(bits))
    del g
    torch.cuda.synchronize()
