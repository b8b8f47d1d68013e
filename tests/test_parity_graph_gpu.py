"""HIP graph capture: the library's calls recorded with torch.cuda.graph and
replayed.  Calls whose path needs a workspace (the fp32 padded copies,
split-K partials) allocate and free it inside the captured work.  Each graph is
replayed several times, with the program's own eager work and
synchronisations in between, and every replay must equal the eager result bit
for bit (the kernels are deterministic and the path choice is the same)."""
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
    ("f32", (1030, 1100, 1000), "f32_padded"),
    ("f32", (512, 512, 16384), "f32_splitk"),
    ("f16", (512, 512, 512), "f16_mfma"),
    ("f16", (1000, 1030, 1100), "f16_staged"),
    ("f16", (128, 128, 16384), "f16_splitk"),
]


def operands(kind, M, N, K):
    if kind == "f32":
        A, B, _ = inputs.sgemm_operands(M, N, K)
        return (torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV),
                torch.empty(M, N, device=DEV))
    A, B = inputs.hgemm_nt_operands(M, N, K)
    return (torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV),
            torch.empty(M, N, device=DEV, dtype=torch.float16))


def call(kind, A, B, C):
    if kind == "f32":
        dg.gemm_f32(A, B, C, 1.0, 0.0)
    else:
        dg.gemm_f16_nt(A, B, C)


def path(kind, A, B, C):
    return dg.f32_path(A, B, C) if kind == "f32" else dg.f16_nt_path(A, B, C)


@pytest.mark.parametrize("kind,shape,expect", CASES, ids=lambda x: str(x))
def test_graph_replays_equal_eager(kind, shape, expect):
    M, N, K = shape
    print("\n[graph case] %s %s %s" % (kind, shape, expect), flush=True)
    sys.stdout.flush()
    A, B, C = operands(kind, M, N, K)
    assert path(kind, A, B, C) == expect
    call(kind, A, B, C)
    torch.cuda.synchronize()
    eager = C.clone()
    C.fill_(float("nan"))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(kind, A, B, C)
    torch.cuda.synchronize()
    A2, B2, C2 = operands(kind, M, N, K)
    for _ in range(3):
        C.fill_(float("nan"))
        call(kind, A2, B2, C2)            # eager work on other buffers between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        bits = torch.int32 if kind == "f32" else torch.int16
        assert torch.equal(C.view(bits), eager.view(bits))
    assert torch.equal(C2.view(bits), eager.view(bits))
    del g
    torch.cuda.synchronize()
