"""The split-K call that allocates nothing (gemm_f16_nt_splitk_static),
called through the C ABI, against gemm_f16_nt_splitk with a caller workspace:
the same kernels over the same ranges, so the outputs must agree bit for bit.
Two calls in a row share the library's scratch area, the second on a smaller
product; a split too large for the area is refused before any work."""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

import oracle
from dense_gemm_sgemm_amd import inputs
from tolerance import f16_check

torch = pytest.importorskip("torch")
import dense_gemm_sgemm_amd as dg  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def abs16(x: np.ndarray) -> np.ndarray:
    return (x.view(np.uint16) & np.uint16(0x7FFF)).view(np.float16)


def dev(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def static_call(dA, dB, dC, splits, stream):
    """The C entry point itself, through ctypes."""
    lib = dg.load_library()
    M, K = dA.shape
    N = dB.shape[0]
    return lib.gemm_f16_nt_splitk_static(M, N, K, dA.data_ptr(), dA.stride(0), dB.data_ptr(),
                                         dB.stride(0), dC.data_ptr(), dC.stride(0), splits,
                                         ctypes.c_void_p(stream.cuda_stream))


def test_static_scratch_matches_workspace_call():
    # (M, N, K, splits): the first call's partial sums take 16 MiB of the
    # 32 MiB area, the second's 2 MiB (a smaller product, fewer ranges)
    cases = [(512, 1024, 8192, 8), (200, 300, 4097, 0)]
    stream = torch.cuda.current_stream()
    refs, outs, ops = [], [], []
    for (M, N, K, splits) in cases:
        say("[case] static split-K %dx%dx%d splits=%d" % (M, N, K, splits))
        need = dg.splitk_workspace_bytes("f16", M, N, K, splits)
        assert 0 < need <= dg.STATIC_SCRATCH_BYTES
        A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
        dA, dB = dev(A), dev(B)
        ref = torch.full((M, N), float("nan"), device=DEV, dtype=torch.float16)
        ws = torch.empty(need, device=DEV, dtype=torch.uint8)
        dg.gemm_f16_nt_splitk(dA, dB, ref, splits=splits, workspace=ws)
        torch.cuda.synchronize()
        refs.append(ref.cpu().numpy())
        outs.append(torch.full((M, N), float("nan"), device=DEV, dtype=torch.float16))
        ops.append((A, B, dA, dB, splits))
    # two calls in a row on one stream, no synchronisation between them
    for (A, B, dA, dB, splits), out in zip(ops, outs):
        assert static_call(dA, dB, out, splits, stream) == dg.GEMM_OK
    torch.cuda.synchronize()
    for (A, B, dA, dB, splits), out, ref in zip(ops, outs, refs):
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
        f16_check(got, oracle.gemm_f16_nt_exact(A, B), oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))
    # the binding, and a second round of the same calls on the area the
    # previous calls left behind
    for (A, B, dA, dB, splits), out, ref in zip(ops, outs, refs):
        out.fill_(float("nan"))
        dg.gemm_f16_nt_splitk_static(dA, dB, out, splits=splits)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), ref.view(np.uint16))


def test_static_scratch_limit_and_unsplit():
    stream = torch.cuda.current_stream()
    M, N, K = 1024, 1024, 16384
    assert dg.splitk_workspace_bytes("f16", M, N, K, 16) > dg.STATIC_SCRATCH_BYTES
    A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
    dA, dB = dev(A), dev(B)
    dC = torch.full((M, N), 7.0, device=DEV, dtype=torch.float16)
    say("[case] static split-K over the limit %dx%dx%d splits=16" % (M, N, K))
    assert static_call(dA, dB, dC, 16, stream) == dg.GEMM_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert bool((dC == 7.0).all())
    # splits = 1 never splits: the plain kernel, equal to gemm_f16_nt
    say("[case] static split-K unsplit %dx%dx%d" % (M, N, K))
    ref = torch.empty_like(dC)
    dg.gemm_f16_nt(dA, dB, ref)
    assert static_call(dA, dB, dC, 1, stream) == dg.GEMM_OK
    torch.cuda.synchronize()
    assert torch.equal(dC.view(torch.int16), ref.view(torch.int16))
