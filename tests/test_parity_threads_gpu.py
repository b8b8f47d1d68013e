"""Two host threads calling the library at once, each on its own stream:
plain calls (the streaming, edge and register-staged kernels) mixed with
calls that take a workspace (explicit split-K and gemm_ex's transposed
copies, the workspace taken per call from torch's allocator on the thread's
stream).  Every result must equal the one-thread result bit for bit."""
from __future__ import annotations

import threading

import pytest

from dense_gemm_sgemm_amd import inputs

torch = pytest.importorskip("torch")
import dense_gemm_sgemm_amd as dg  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SHAPES = [("f32", (1030, 1100, 1000)), ("f32_splitk", (512, 512, 16384)),
          ("f16", (1000, 1030, 1100)), ("f16_splitk", (128, 128, 16384)),
          ("f32", (1024, 1024, 1024)), ("ex_nn", (500, 301, 153)), ("ex_nn", (1000, 1030, 1100)),
          ("ex_nn", (2048, 2304, 768))]   # the last read in place, no workspace


def make(kind, M, N, K):
    if kind.startswith("f32"):
        A, B, _ = inputs.sgemm_operands(M, N, K)
        return torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV), torch.float32
    A, B = inputs.hgemm_nt_operands(M, N, K)
    dA, dB = torch.from_numpy(A).to(DEV), torch.from_numpy(B).to(DEV)
    if kind == "ex_nn":
        dB = dB.t().contiguous()            # B stored K x N
    return dA, dB, torch.float16


def run(kind, A, B, C, stream):
    if kind == "f32":
        dg.gemm_f32(A, B, C, 1.0, 0.0, stream=stream)
    elif kind == "f32_splitk":
        dg.gemm_f32_splitk(A, B, C, 1.0, 0.0, stream=stream)
    elif kind == "f16_splitk":
        dg.gemm_f16_nt_splitk(A, B, C, stream=stream)
    elif kind == "ex_nn":
        dg.gemm_ex(A, B, C, "n", "n", stream=stream)
    else:
        dg.gemm_f16_nt(A, B, C, stream=stream)


def test_two_threads_two_streams():
    ops = [(kind, M, N) + make(kind, M, N, K) for kind, (M, N, K) in SHAPES]
    ref = []
    for kind, M, N, A, B, dt in ops:
        C = torch.empty(M, N, device=DEV, dtype=dt)
        run(kind, A, B, C, None)
        ref.append(C)
    torch.cuda.synchronize()
    rounds = 6
    outs = {t: [[torch.full((M, N), float("nan"), device=DEV, dtype=dt) for (kind, M, N, A, B, dt) in ops]
                for _ in range(rounds)] for t in range(2)}
    errors = []

    def worker(t):
        try:
            s = torch.cuda.Stream()   # default priority
            for r in range(rounds):
                order = range(len(ops)) if (r + t) % 2 == 0 else reversed(range(len(ops)))
                for i in order:
                    kind, M, N, A, B, dt = ops[i]
                    run(kind, A, B, outs[t][r][i], s)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(2):
        for r in range(rounds):
            for i, (kind, M, N, A, B, dt) in enumerate(ops):
                bits = torch.int32 if dt == torch.float32 else torch.int16
                assert torch.equal(outs[t][r][i].view(bits), ref[i].view(bits)), (t, r, kind, M, N)
