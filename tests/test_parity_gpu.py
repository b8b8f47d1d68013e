"""GPU parity: the HIP kernels, called through the C ABI, against the CPU oracle.

Every configuration of the hot path (256^3, 1024^3 and 4096^3 fp32 at beta 0
and 0.5; 5376x5376x2048 and 5000x3001x1537 fp16) is compared element by
element with the full oracle result, and so are the small and medium shapes.
Only some secondary large shapes (the fp32 streaming-kernel sweeps) are
compared on sampled outputs that the oracle computes one by one: whole rows,
whole columns, whole output tiles (first, last and one in the middle) and
random points.  Tolerances are in ``tolerance.py``.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from dense_gemm_sgemm_amd import inputs
from expect import expected_f16_path, expected_f32_path
from tolerance import f16_check, f16_ex_check, f32_check, f32_tolerance

torch = pytest.importorskip("torch")
import dense_gemm_sgemm_amd as dg  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _announce(request):
    say("\n[gpu case] %s" % request.node.nodeid)
    yield


@pytest.fixture(params=["auto", "general"])
def path_mode(request, monkeypatch):
    if request.param == "general":
        monkeypatch.setenv("MI355GEMM_FORCE_PATH", "general")
    else:
        monkeypatch.delenv("MI355GEMM_FORCE_PATH", raising=False)
    return request.param


def dev(x: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def gpu_f32(A, B, alpha=1.0, beta=0.0, C=None, expect=None):
    dA, dB = dev(A), dev(B)
    M, N = A.shape[0], B.shape[1]
    dC = dev(C) if C is not None else torch.full((M, N), float("nan"), device=DEV)
    if expect is not None:
        assert dg.f32_path(dA, dB, dC, alpha, beta) == expect
    dg.gemm_f32(dA, dB, dC, alpha, beta)
    torch.cuda.synchronize()
    return dC.cpu().numpy()


def gpu_f16(A, B, expect=None):
    dA, dB = dev(A), dev(B)
    dC = torch.full((A.shape[0], B.shape[0]), float("nan"), device=DEV, dtype=torch.float16)
    if expect is not None:
        assert dg.f16_nt_path(dA, dB, dC) == expect
    dg.gemm_f16_nt(dA, dB, dC)
    torch.cuda.synchronize()
    return dC.cpu().numpy()


def abs16(x: np.ndarray) -> np.ndarray:
    return (x.view(np.uint16) & np.uint16(0x7FFF)).view(np.float16)


# ----------------------------------------------------------------- fp32 -----
F32_SHAPES = [(1, 1, 1), (3, 5, 7), (17, 33, 9), (64, 64, 16), (65, 63, 17), (128, 128, 16),
              (128, 256, 32), (256, 128, 48), (129, 127, 31), (256, 384, 160), (200, 300, 1),
              (384, 256, 512), (192, 320, 48), (1000, 700, 333), (2048, 2112, 64),
              (4160, 4096, 32)]


@pytest.mark.parametrize("shape", F32_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_shapes(shape, path_mode):
    M, N, K = shape
    A, B, _ = inputs.sgemm_operands(M, N, K)
    got = gpu_f32(A, B, expect=expected_f32_path(path_mode, M, N, K))
    f32_check(got, oracle.gemm_f32(A, B), f32_tolerance(K, 1.0, 1.0))


@pytest.mark.parametrize("beta", [0.0, 0.5, -1.25])
@pytest.mark.parametrize("alpha", [1.0, 2.0, -0.5])
def test_f32_alpha_beta(alpha, beta, path_mode):
    M, N, K = 256, 256, 64
    A, B, C = inputs.sgemm_operands(M, N, K, with_c=True)
    got = gpu_f32(A, B, alpha, beta, C.copy())
    ref = oracle.gemm_f32(A, B, alpha, beta, C)
    f32_check(got, ref, f32_tolerance(K, 1.0, 1.0, alpha, beta, 1.0))


def test_f32_beta_zero_ignores_nan_and_alpha_scales_exactly(path_mode):
    M, N, K = 256, 128, 96
    A, B, _ = inputs.sgemm_operands(M, N, K)
    one = gpu_f32(A, B, 1.0, 0.0)                       # C prefilled with NaN
    assert np.all(np.isfinite(one))
    two = gpu_f32(A, B, 2.0, 0.0)
    assert np.array_equal(two, 2.0 * one)


def test_f32_quick_returns():
    M, N = 64, 96
    A, B, C = inputs.sgemm_operands(M, N, 16, with_c=True)
    got = gpu_f32(A, B, 0.0, 0.5, C.copy(), expect="f32_scale")
    assert np.array_equal(got, (np.float32(0.5) * C))
    got = gpu_f32(A[:, :0], B[:0, :], 1.0, 0.0, None, expect="f32_scale")
    assert np.array_equal(got, np.zeros((M, N), np.float32))
    dA = torch.zeros(0, 5, device=DEV)
    dB = torch.zeros(5, 7, device=DEV)
    dC = torch.zeros(0, 7, device=DEV)
    dg.gemm_f32(dA, dB, dC)                             # M == 0: no-op
    torch.cuda.synchronize()


def test_f32_small_integers_are_exact(path_mode):
    for (M, N, K) in [(128, 128, 512), (77, 65, 300)]:
        A = inputs.small_ints((M, K), 1, -3, 3, np.float32)
        B = inputs.small_ints((K, N), 2, -3, 3, np.float32)
        got = gpu_f32(A, B)
        assert np.array_equal(got.astype(np.float64), oracle.gemm_f32(A, B))


def test_f32_padded_leading_dimensions(path_mode):
    M, N, K = 256, 256, 64
    for pad in (3, 8):
        Abig, Bbig, Cbig = inputs.sgemm_operands(M, N + pad, K + pad, with_c=True)
        A, B = Abig[:, :K], Bbig[:K, :N]
        dA, dB, dC = dev(Abig)[:, :K], dev(Bbig)[:K, :N], dev(Cbig)
        dCv = dC[:, :N]
        dg.gemm_f32(dA, dB, dCv, 1.0, 0.5)
        torch.cuda.synchronize()
        got = dC.cpu().numpy()
        ref = oracle.gemm_f32(A, B, 1.0, 0.5, Cbig[:, :N])
        f32_check(got[:, :N], ref, f32_tolerance(K, 1.0, 1.0, 1.0, 0.5, 1.0))
        assert np.array_equal(got[:, N:], Cbig[:, N:])   # the padding is not written


def test_f32_unaligned_operands(path_mode):
    """A, B and C starting one float into their buffers with odd leading
    dimensions, K and N tails of every length modulo 4; C outside its window
    stays untouched, beta = 0.5 reads only the window."""
    for (M, N, K) in [(133, 70, 45), (260, 129, 67), (64, 200, 130), (5, 301, 9)]:
        lda, ldb, ldc = K + 3, N + 1, N + 5
        A, B, C = inputs.sgemm_operands(M, N, K, with_c=True, dist="normal")
        bufA = torch.zeros(M * lda + 2, device=DEV)
        bufB = torch.zeros(K * ldb + 2, device=DEV)
        bufC = torch.full((M * ldc + 2,), 5.0, device=DEV)
        dA = bufA[1:1 + M * lda].view(M, lda)[:, :K]
        dB = bufB[1:1 + K * ldb].view(K, ldb)[:, :N]
        dC = bufC[1:1 + M * ldc].view(M, ldc)[:, :N]
        dA.copy_(dev(A))
        dB.copy_(dev(B))
        dC.copy_(dev(C))
        assert dg.f32_path(dA, dB, dC, 1.0, 0.5) == "f32_general"
        dg.gemm_f32(dA, dB, dC, 1.0, 0.5)
        torch.cuda.synchronize()
        tol = f32_tolerance(K, np.abs(A).max(), np.abs(B).max(), 1.0, 0.5, np.abs(C).max())
        f32_check(dC.cpu().numpy(), oracle.gemm_f32(A, B, 1.0, 0.5, C), tol)
        full = bufC.cpu().numpy()
        mask = np.ones(full.shape, bool)
        idx = 1 + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
        mask[idx.ravel()] = False
        assert np.all(full[mask] == 5.0)


def test_f32_deterministic():
    A, B, _ = inputs.sgemm_operands(512, 512, 256)
    assert np.array_equal(gpu_f32(A, B), gpu_f32(A, B))


def test_f32_on_a_side_stream():
    A, B, _ = inputs.sgemm_operands(256, 256, 128)
    s = torch.cuda.Stream()
    dA, dB = dev(A), dev(B)
    dC = torch.empty(256, 256, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        dg.gemm_f32(dA, dB, dC)
    s.synchronize()
    f32_check(dC.cpu().numpy(), oracle.gemm_f32(A, B), f32_tolerance(128, 1.0, 1.0))


# ----------------------------------------------------------------- fp16 -----
# Includes shapes for both fast-path tile widths (N % 256 == 0 and N % 224 == 0),
# a single K slab, and several tiles in each direction.
F16_SHAPES = [(1, 1, 1), (3, 5, 7), (17, 33, 9), (64, 64, 32), (65, 63, 33), (256, 256, 64),
              (256, 512, 128), (512, 256, 192), (257, 255, 65), (300, 200, 1), (512, 768, 320),
              (129, 130, 1537), (256, 224, 64), (512, 448, 128), (768, 672, 256), (256, 1792, 576),
              (128, 128, 64), (384, 640, 192), (1152, 896, 448)]


@pytest.mark.parametrize("shape", F16_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f16_shapes(shape, path_mode):
    M, N, K = shape
    A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
    got = gpu_f16(A, B, expect=expected_f16_path(path_mode, M, N, K))
    ref = oracle.gemm_f16_nt_exact(A, B)
    sab = oracle.gemm_f16_nt_exact(abs16(A), abs16(B))
    f16_check(got, ref, sab)


def test_f16_small_integers_are_exact_and_ties_go_even(path_mode):
    A = inputs.small_ints((256, 512), 1, -2, 2, np.float16)
    B = inputs.small_ints((256, 512), 2, -2, 2, np.float16)
    got = gpu_f16(A, B)
    exact = A.astype(np.int64) @ B.astype(np.int64).T
    assert np.array_equal(got.view(np.uint16), exact.astype(np.float16).view(np.uint16))
    # sums past 2048: ties go to the even neighbour, as in the oracle's pins
    K = 2112
    A = np.zeros((256, K), np.float16)
    B = np.zeros((256, K), np.float16)
    B[:, :] = 1.0
    for row, total in enumerate([2049, 2050, 2051, 2053, 2047, 4097]):
        A[row, :min(total, K)] = 1.0
        if total > K:
            A[row, 0] = total - (K - 1)
    got = gpu_f16(A, B)
    _, want = oracle.gemm_f16_nt(A, B)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))
    assert list(got[:6, 0].astype(np.float64)) == [2048.0, 2050.0, 2052.0, 2052.0, 2047.0, 4096.0]


def test_f16_outer_product_rounding(path_mode):
    """Only k = 0 is nonzero: fp32 holds a*b exactly, so C must equal half(a*b)."""
    rng = np.random.default_rng(21)
    M, N, K = 256, 256, 64
    A = np.zeros((M, K), np.float16)
    B = np.zeros((N, K), np.float16)
    A[:, 0] = rng.normal(0, 20, M).astype(np.float16)
    B[:, 0] = rng.normal(0, 0.05, N).astype(np.float16)
    got = gpu_f16(A, B)
    _, want = oracle.gemm_f16_nt(A, B)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_f16_quick_returns():
    dA = torch.zeros(64, 0, device=DEV, dtype=torch.float16)
    dB = torch.zeros(32, 0, device=DEV, dtype=torch.float16)
    dC = torch.full((64, 32), 7.0, device=DEV, dtype=torch.float16)
    assert dg.f16_nt_path(dA, dB, dC) == "f16_zero"
    dg.gemm_f16_nt(dA, dB, dC)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dC).item() == 0


def test_f16_padded_leading_dimensions(path_mode):
    M, N, K = 256, 256, 128
    for pad in (1, 8):
        Abig, Bbig = inputs.hgemm_nt_operands(M, N, K + pad)
        dA, dB = dev(Abig)[:, :K], dev(Bbig)[:, :K]
        dC = torch.full((M, N + pad), 3.0, device=DEV, dtype=torch.float16)
        dg.gemm_f16_nt(dA, dB, dC[:, :N])
        torch.cuda.synchronize()
        got = dC.cpu().numpy()
        A, B = Abig[:, :K], Bbig[:, :K]
        f16_check(got[:, :N], oracle.gemm_f16_nt_exact(A, B),
                  oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))
        assert np.all(got[:, N:] == 3.0)


def test_f16_unaligned_operands(path_mode):
    """Operands and C starting one element into their buffers, odd leading
    dimensions and K tails of every length modulo 8: rows start at arbitrary
    2-byte addresses, and the row ends fall inside 16-byte chunks."""
    for (M, N, K) in [(133, 70, 45), (260, 129, 67), (64, 200, 130), (5, 300, 9)]:
        lda, ldb, ldc = K + 3, K + 1, N + 5
        A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
        bufA = torch.zeros(M * lda + 2, device=DEV, dtype=torch.float16)
        bufB = torch.zeros(N * ldb + 2, device=DEV, dtype=torch.float16)
        bufC = torch.full((M * ldc + 2,), 5.0, device=DEV, dtype=torch.float16)
        dA = bufA[1:1 + M * lda].view(M, lda)[:, :K]
        dB = bufB[1:1 + N * ldb].view(N, ldb)[:, :K]
        dC = bufC[1:1 + M * ldc].view(M, ldc)[:, :N]
        dA.copy_(dev(A))
        dB.copy_(dev(B))
        assert dg.f16_nt_path(dA, dB, dC) == (
            "f16_gemv" if path_mode == "auto" and min(M, N) <= 8 else "f16_general")
        dg.gemm_f16_nt(dA, dB, dC)
        torch.cuda.synchronize()
        f16_check(dC.cpu().numpy(), oracle.gemm_f16_nt_exact(A, B),
                  oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))
        # everything outside C's M x N window is untouched
        full = bufC.cpu().numpy()
        mask = np.ones(full.shape, bool)
        idx = 1 + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
        mask[idx.ravel()] = False
        assert np.all(full[mask] == 5.0)


def test_f16_transpose_relation_and_determinism():
    """C(B, A) is C(A, B) transposed: both match the oracle, and runs repeat bitwise."""
    A, B = inputs.hgemm_nt_operands(512, 256, 256)
    c1 = gpu_f16(A, B)
    assert np.array_equal(c1.view(np.uint16), gpu_f16(A, B).view(np.uint16))
    ct = gpu_f16(B, A)
    ref = oracle.gemm_f16_nt_exact(A, B)
    sab = oracle.gemm_f16_nt_exact(abs16(A), abs16(B))
    f16_check(c1, ref, sab)
    f16_check(ct.T, ref, sab)


# ------------------------------------------------- fused write-back ------
EPI_CASES = [("none", True, False), ("relu", True, True), ("silu", True, True),
             ("silu", False, True), ("relu", False, False), ("none", False, False)]
EPI_SHAPES = [(256, 224, 64), (512, 448, 128), (256, 512, 192), (133, 70, 45), (257, 255, 65)]


def epi_operands(M, N, K, use_bias, use_res, seed=40):
    A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
    rng = np.random.default_rng(seed)
    bias = rng.normal(0, 1.5, N).astype(np.float16) if use_bias else None
    res = rng.normal(0, 2.0, (M, N)).astype(np.float16) if use_res else None
    return A, B, bias, res


def check_ex(got, A, B, bias, act, res):
    ref = oracle.gemm_f16_nt_ex_exact(A, B, bias, act, res)
    sab = oracle.gemm_f16_nt_exact(abs16(A), abs16(B))
    babs = 0.0 if bias is None else np.abs(bias.astype(np.float64))[None, :]
    rabs = 0.0 if res is None else np.abs(res.astype(np.float64))
    return f16_ex_check(got, ref, sab, babs, rabs)


@pytest.mark.parametrize("act,use_bias,use_res", EPI_CASES)
@pytest.mark.parametrize("shape", EPI_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f16_fused_epilogue(shape, act, use_bias, use_res, path_mode):
    M, N, K = shape
    A, B, bias, res = epi_operands(M, N, K, use_bias, use_res)
    dA, dB = dev(A), dev(B)
    dbias = dev(bias) if bias is not None else None
    dres = dev(res) if res is not None else None
    dC = torch.full((M, N), float("nan"), device=DEV, dtype=torch.float16)
    want = expected_f16_path(path_mode, M, N, K).replace("f16_zero", "f16_general")
    assert dg.f16_nt_ex_path(dA, dB, dC, dbias, act, dres) == want
    dg.gemm_f16_nt_ex(dA, dB, dC, dbias, act, dres)
    torch.cuda.synchronize()
    check_ex(dC.cpu().numpy(), A, B, bias, act, res)


def test_f16_fused_in_place_residual_and_saturation(path_mode):
    """residual = C (in place), biases far out in SiLU's tails, and K = 0."""
    M, N, K = 512, 448, 128
    A, B, _, res = epi_operands(M, N, K, False, True)
    bias = np.linspace(-30, 30, N).astype(np.float16)
    dC = dev(res)
    dg.gemm_f16_nt_ex(dev(A), dev(B), dC, dev(bias), "silu", dC)
    torch.cuda.synchronize()
    check_ex(dC.cpu().numpy(), A, B, bias, "silu", res)
    # K = 0: C = act(bias) + residual
    Z = np.zeros((M, 0), np.float16)
    Zb = np.zeros((N, 0), np.float16)
    dC = torch.full((M, N), float("nan"), device=DEV, dtype=torch.float16)
    dg.gemm_f16_nt_ex(dev(Z), dev(Zb), dC, dev(bias), "relu", dev(res))
    torch.cuda.synchronize()
    check_ex(dC.cpu().numpy(), Z, Zb, bias, "relu", res)


def test_f16_fused_unaligned_bias_and_residual():
    """bias one element into its buffer and residual rows of odd length: the
    fused call still runs, on the edge kernel."""
    M, N, K = 256, 224, 64
    A, B, bias, res = epi_operands(M, N, K, True, True)
    bbuf = torch.zeros(N + 1, device=DEV, dtype=torch.float16)
    bbuf[1:].copy_(dev(bias))
    rbuf = torch.zeros(M, N + 1, device=DEV, dtype=torch.float16)
    rbuf[:, :N].copy_(dev(res))
    dA, dB = dev(A), dev(B)
    dC = torch.empty(M, N, device=DEV, dtype=torch.float16)
    assert dg.f16_nt_ex_path(dA, dB, dC, bbuf[1:], "silu", rbuf[:, :N]) == "f16_general"
    dg.gemm_f16_nt_ex(dA, dB, dC, bbuf[1:], "silu", rbuf[:, :N])
    torch.cuda.synchronize()
    check_ex(dC.cpu().numpy(), A, B, bias, "silu", res)


def test_workload_hgemm_fused():
    """5376 x 5376 x 2048 with bias, SiLU and residual on the fast kernel,
    every output against the oracle."""
    M, N, K = 5376, 5376, 2048
    A, B = inputs.workload_operands("hgemm_nt_5376x5376x2048")
    rng = np.random.default_rng(41)
    bias = rng.normal(0, 4.0, N).astype(np.float16)
    res = rng.normal(0, 4.0, (M, N)).astype(np.float16)
    dC = torch.empty(M, N, device=DEV, dtype=torch.float16)
    dA, dB, dbias, dres = dev(A), dev(B), dev(bias), dev(res)
    assert dg.f16_nt_ex_path(dA, dB, dC, dbias, "silu", dres) == "f16_mfma"
    dg.gemm_f16_nt_ex(dA, dB, dC, dbias, "silu", dres)
    torch.cuda.synchronize()
    got = dC.cpu().numpy()
    ref = oracle.gemm_f16_nt_ex_exact(A, B, bias, "silu", res)
    sab = oracle.gemm_f16_nt_exact(abs16(A), abs16(B))
    r = f16_ex_check(got, ref, sab, np.abs(bias.astype(np.float64))[None, :],
                     np.abs(res.astype(np.float64)))
    say("[fused 5376x5376x2048 silu] checked all %d outputs, max %.2f ulp"
        % (r["count"], r["max_ulps"]))


# ---------------------------------------------------- matrix-vector -------
# M or N at most 8: one operand is streamed once and the other is a few
# vectors.  Long rows (K >= 4096) are split over a workgroup, shorter ones over
# a wave; K tails of every length modulo 8; M < N and N < M orientations.
GEMV_SHAPES = [(1, 1, 1), (1, 7, 5), (1, 300, 9), (1, 1000, 4096), (1, 777, 4103),
               (1, 513, 8192), (2, 300, 2055), (3, 129, 63), (8, 1030, 4096), (4, 64, 520),
               (6, 70, 12345), (300, 1, 9), (1000, 1, 4096), (777, 3, 4103), (129, 8, 300),
               (5, 7, 100), (7, 5, 100), (8, 8, 4100), (1, 2, 33001), (2, 100, 9001),
               (1, 64, 2048), (3, 40, 1536)]


@pytest.mark.parametrize("shape", GEMV_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f16_gemv_shapes(shape, path_mode):
    M, N, K = shape
    A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
    got = gpu_f16(A, B, expect=expected_f16_path(path_mode, M, N, K))
    f16_check(got, oracle.gemm_f16_nt_exact(A, B), oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))


def test_f16_gemv_strided_and_unaligned():
    """Vectors and matrix rows at odd 2-byte offsets with padded leading
    dimensions, and a C column written with stride ldc: nothing outside C's
    window changes."""
    for (M, N, K) in [(1, 500, 4099), (3, 200, 777), (500, 1, 4099), (200, 5, 777)]:
        lda, ldb, ldc = K + 3, K + 1, N + 5
        A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
        bufA = torch.zeros(M * lda + 2, device=DEV, dtype=torch.float16)
        bufB = torch.zeros(N * ldb + 2, device=DEV, dtype=torch.float16)
        bufC = torch.full((M * ldc + 2,), 5.0, device=DEV, dtype=torch.float16)
        dA = bufA[1:1 + M * lda].view(M, lda)[:, :K]
        dB = bufB[1:1 + N * ldb].view(N, ldb)[:, :K]
        dC = bufC[1:1 + M * ldc].view(M, ldc)[:, :N]
        dA.copy_(dev(A))
        dB.copy_(dev(B))
        assert dg.f16_nt_path(dA, dB, dC) == "f16_gemv"
        dg.gemm_f16_nt(dA, dB, dC)
        torch.cuda.synchronize()
        f16_check(dC.cpu().numpy(), oracle.gemm_f16_nt_exact(A, B),
                  oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))
        full = bufC.cpu().numpy()
        mask = np.ones(full.shape, bool)
        idx = 1 + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
        mask[idx.ravel()] = False
        assert np.all(full[mask] == 5.0)


def test_f16_gemv_exact_cases_and_determinism():
    """Small-integer products are exact, sums past 2048 round ties to even,
    and repeated runs agree bitwise."""
    A = inputs.small_ints((1, 4096), 1, -2, 2, np.float16)
    B = inputs.small_ints((3000, 4096), 2, -2, 2, np.float16)
    got = gpu_f16(A, B, expect="f16_gemv")
    exact = A.astype(np.int64) @ B.astype(np.int64).T
    assert np.array_equal(got.view(np.uint16), exact.astype(np.float16).view(np.uint16))
    got_t = gpu_f16(B, A, expect="f16_gemv")
    assert np.array_equal(got_t.T.view(np.uint16), got.view(np.uint16))
    K = 4352
    A = np.ones((1, K), np.float16)
    B = np.zeros((6, K), np.float16)
    for row, total in enumerate([2049, 2050, 2051, 2053, 2047, 4097]):
        B[row, :total] = 1.0
    got = gpu_f16(A, B, expect="f16_gemv")
    assert list(got[0].astype(np.float64)) == [2048.0, 2050.0, 2052.0, 2052.0, 2047.0, 4096.0]
    A, B = inputs.hgemm_nt_operands(4, 3000, 5000, dist="normal")
    assert np.array_equal(gpu_f16(A, B).view(np.uint16), gpu_f16(A, B).view(np.uint16))


GEMV_EPI_SHAPES = [(1, 300, 4096), (4, 129, 1000), (300, 2, 520), (1, 1000, 8200), (9, 8, 77)]


@pytest.mark.parametrize("act,use_bias,use_res", EPI_CASES)
@pytest.mark.parametrize("shape", GEMV_EPI_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f16_gemv_fused_epilogue(shape, act, use_bias, use_res):
    M, N, K = shape
    A, B, bias, res = epi_operands(M, N, K, use_bias, use_res)
    dA, dB = dev(A), dev(B)
    dbias = dev(bias) if bias is not None else None
    dres = dev(res) if res is not None else None
    dC = torch.full((M, N), float("nan"), device=DEV, dtype=torch.float16)
    assert dg.f16_nt_ex_path(dA, dB, dC, dbias, act, dres) == "f16_gemv"
    dg.gemm_f16_nt_ex(dA, dB, dC, dbias, act, dres)
    torch.cuda.synchronize()
    check_ex(dC.cpu().numpy(), A, B, bias, act, res)


def test_f16_gemv_fused_in_place_and_unaligned():
    """residual = C in place, bias one element into its buffer, for both
    orientations."""
    for (M, N, K) in [(1, 1000, 4096), (700, 3, 999)]:
        A, B, _, res = epi_operands(M, N, K, False, True)
        bias = np.linspace(-30, 30, N).astype(np.float16)
        bbuf = torch.zeros(N + 1, device=DEV, dtype=torch.float16)
        bbuf[1:].copy_(dev(bias))
        dC = dev(res)
        assert dg.f16_nt_ex_path(dev(A), dev(B), dC, bbuf[1:], "silu", dC) == "f16_gemv"
        dg.gemm_f16_nt_ex(dev(A), dev(B), dC, bbuf[1:], "silu", dC)
        torch.cuda.synchronize()
        check_ex(dC.cpu().numpy(), A, B, bias, "silu", res)


def test_f16_gemv_many_launches():
    """2^24 + 37 rows of 8: more row groups than one launch takes, so the
    rows are split over two launches."""
    M, N, K = 1, (1 << 24) + 37, 8
    A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
    got = gpu_f16(A, B, expect="f16_gemv")
    rows = np.zeros(200000, np.int32)
    cols = np.concatenate([np.arange(100000), np.arange(N - 100000, N)]).astype(np.int32)
    ref = oracle.gemm_f16_nt_points(A, B, rows, cols)
    sab = oracle.gemm_f16_nt_points(abs16(A), abs16(B), rows, cols)
    f16_check(got[rows, cols], ref, sab)
    j = np.random.default_rng(5).integers(0, N, 100000).astype(np.int32)
    f16_check(got[0, j], oracle.gemm_f16_nt_points(A, B, np.zeros_like(j), j),
              oracle.gemm_f16_nt_points(abs16(A), abs16(B), np.zeros_like(j), j))


def test_workload_hgemv_decode():
    """The 1 x 16384 x 4096 decode product, every output checked."""
    A, B = inputs.workload_operands("hgemv_nt_1x16384x4096")
    got = gpu_f16(A, B, expect="f16_gemv")
    res = f16_check(got, oracle.gemm_f16_nt_exact(A, B),
                    oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))
    say("[hgemv_nt_1x16384x4096] checked %d outputs, max %.2f ulp, literal-2ulp violations %d"
        % (res["count"], res["max_ulps"], res["literal_2ulp_violations"]))


# ----------------------------------------------------------- split-K -------
# Long K over few output tiles: K cut into ranges whose fp32 partial sums are
# added in a fixed order.  Automatic (through gemm_f16_nt / gemm_f32, with a
# stream-ordered workspace) and explicit (caller's split count and workspace).
SPLITK_SHAPES = [(128, 128, 16384), (512, 512, 16384), (300, 200, 5000), (1000, 700, 3001),
                 (136, 264, 2111), (64, 1000, 4099)]


def gpu_f16_splitk(A, B, splits=0):
    """gemm_f16_nt_splitk with the binding's own workspace; asserts that the
    library's rule splits these sizes when splits <= 0."""
    M, N, K = A.shape[0], B.shape[0], A.shape[1]
    if splits <= 0:
        assert dg.splitk_workspace_bytes("f16", M, N, K, 0) > 0
    dC = torch.full((M, N), float("nan"), device=DEV, dtype=torch.float16)
    dg.gemm_f16_nt_splitk(dev(A), dev(B), dC, splits=splits)
    torch.cuda.synchronize()
    return dC.cpu().numpy()


@pytest.mark.parametrize("shape", SPLITK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f16_splitk_auto(shape):
    M, N, K = shape
    A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
    got = gpu_f16_splitk(A, B)
    f16_check(got, oracle.gemm_f16_nt_exact(A, B), oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
def test_f16_splitk_explicit(splits):
    for (M, N, K) in [(256, 384, 4096), (133, 70, 1045), (9, 300, 777)]:
        A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
        dA, dB = dev(A), dev(B)
        dC = torch.full((M, N), float("nan"), device=DEV, dtype=torch.float16)
        dg.gemm_f16_nt_splitk(dA, dB, dC, splits=splits)
        torch.cuda.synchronize()
        f16_check(dC.cpu().numpy(), oracle.gemm_f16_nt_exact(A, B),
                  oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))


def test_f16_splitk_unaligned_workspace_reuse_and_determinism():
    """Operands at odd offsets with padded rows, a C window inside a larger
    buffer, one workspace reused by two calls in a row (the second smaller),
    and repeated runs bitwise equal."""
    ws = torch.empty(dg.splitk_workspace_bytes("f16", 300, 200, 5001, 9), dtype=torch.uint8,
                     device=DEV)
    for (M, N, K, splits) in [(300, 200, 5001, 9), (133, 70, 2049, 4)]:
        lda, ldb, ldc = K + 3, K + 1, N + 5
        A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
        bufA = torch.zeros(M * lda + 2, device=DEV, dtype=torch.float16)
        bufB = torch.zeros(N * ldb + 2, device=DEV, dtype=torch.float16)
        bufC = torch.full((M * ldc + 2,), 5.0, device=DEV, dtype=torch.float16)
        dA = bufA[1:1 + M * lda].view(M, lda)[:, :K]
        dB = bufB[1:1 + N * ldb].view(N, ldb)[:, :K]
        dC = bufC[1:1 + M * ldc].view(M, ldc)[:, :N]
        dA.copy_(dev(A))
        dB.copy_(dev(B))
        assert dg.splitk_workspace_bytes("f16", M, N, K, splits) <= ws.numel()
        dg.gemm_f16_nt_splitk(dA, dB, dC, splits=splits, workspace=ws)
        torch.cuda.synchronize()
        first = bufC.cpu().numpy()
        f16_check(dC.cpu().numpy(), oracle.gemm_f16_nt_exact(A, B),
                  oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))
        mask = np.ones(first.shape, bool)
        idx = 1 + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
        mask[idx.ravel()] = False
        assert np.all(first[mask] == 5.0)
        dg.gemm_f16_nt_splitk(dA, dB, dC, splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(bufC.cpu().numpy().view(np.uint16), first.view(np.uint16))


def test_splitk_binding_workspace_on_a_side_stream():
    """The binding's own workspace (workspace=None) for calls on a side stream:
    right after each call the current stream allocates and fills tensors of
    the workspace's size, which must not disturb the side stream's partial
    sums; then both results are checked against the oracle."""
    side = torch.cuda.Stream()
    M, N, K = 256, 384, 8192
    A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
    A32, B32, _ = inputs.sgemm_operands(M, N, K)
    dA, dB, dA32, dB32 = dev(A), dev(B), dev(A32), dev(B32)
    dC = torch.full((M, N), float("nan"), device=DEV, dtype=torch.float16)
    dC32 = torch.full((M, N), float("nan"), device=DEV)
    torch.cuda.synchronize()
    need16 = dg.splitk_workspace_bytes("f16", M, N, K, 8)
    need32 = dg.splitk_workspace_bytes("f32", M, N, K, 8)
    assert need16 > 0 and need32 > 0
    dg.gemm_f16_nt_splitk(dA, dB, dC, splits=8, stream=side)
    junk16 = torch.empty(need16 // 4, device=DEV)
    junk16.fill_(float("nan"))
    dg.gemm_f32_splitk(dA32, dB32, dC32, splits=8, stream=side)
    junk32 = torch.empty(need32 // 4, device=DEV)
    junk32.fill_(float("nan"))
    torch.cuda.synchronize()
    f16_check(dC.cpu().numpy(), oracle.gemm_f16_nt_exact(A, B),
              oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))
    f32_check(dC32.cpu().numpy(), oracle.gemm_f32(A32, B32), f32_tolerance(K, 1.0, 1.0))
    del junk16, junk32


@pytest.mark.parametrize("shape", [(512, 448, 8192), (300, 200, 5000)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("act,use_bias,use_res", EPI_CASES[:4])
def test_f16_splitk_fused(shape, act, use_bias, use_res):
    """The fused write-back on gemm_ex's split-K path (the binding passes a
    workspace of the size query's bytes), in place when there is a residual."""
    M, N, K = shape
    A, B, bias, res = epi_operands(M, N, K, use_bias, use_res)
    dA, dB = dev(A), dev(B)
    dbias = dev(bias) if bias is not None else None
    dres = dev(res) if res is not None else None
    dC = dres if dres is not None else torch.full((M, N), float("nan"), device=DEV,
                                                  dtype=torch.float16)
    assert dg.ex_path(dA, dB, dC, "n", "t", dbias, act, dres) == "f16_splitk"
    assert dg.f16_nt_ex_path(dA, dB, dC, dbias, act, dres) != "f16_splitk"
    dg.gemm_ex(dA, dB, dC, "n", "t", dbias, act, dres)
    torch.cuda.synchronize()
    check_ex(dC.cpu().numpy(), A, B, bias, act, res)


F32_SPLITK_SHAPES = [(512, 512, 16384), (100, 70, 3000), (300, 257, 4099), (128, 384, 2048)]


@pytest.mark.parametrize("beta", [0.0, 0.5])
@pytest.mark.parametrize("shape", F32_SPLITK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_splitk_auto(shape, beta):
    M, N, K = shape
    A, B, C = inputs.sgemm_operands(M, N, K, with_c=True)
    assert dg.splitk_workspace_bytes("f32", M, N, K, 0) > 0
    dC = dev(C)
    dg.gemm_f32_splitk(dev(A), dev(B), dC, 1.0, beta)
    torch.cuda.synchronize()
    got = dC.cpu().numpy()
    tol = f32_tolerance(K, np.abs(A).max(), np.abs(B).max(), 1.0, beta, np.abs(C).max())
    f32_check(got, oracle.gemm_f32(A, B, 1.0, beta, C), tol)


@pytest.mark.parametrize("splits", [1, 2, 5, 33])
def test_f32_splitk_explicit(splits):
    for (M, N, K, alpha, beta) in [(256, 256, 4096, -0.5, 1.25), (133, 70, 1043, 2.0, 0.0),
                                   (64, 200, 530, 1.0, -1.0)]:
        A, B, C = inputs.sgemm_operands(M, N, K, with_c=True, dist="normal")
        dA, dB, dC = dev(A), dev(B), dev(C)
        dg.gemm_f32_splitk(dA, dB, dC, alpha, beta, splits=splits)
        torch.cuda.synchronize()
        tol = f32_tolerance(K, np.abs(A).max(), np.abs(B).max(), alpha, beta, np.abs(C).max())
        f32_check(dC.cpu().numpy(), oracle.gemm_f32(A, B, alpha, beta, C), tol)


def test_f32_splitk_beta_zero_ignores_nan_and_repeats():
    A, B, _ = inputs.sgemm_operands(512, 512, 16384)

    def run():
        dC = torch.full((512, 512), float("nan"), device=DEV)
        dg.gemm_f32_splitk(dev(A), dev(B), dC, 1.0, 0.0)
        torch.cuda.synchronize()
        return dC.cpu().numpy()
    one = run()
    assert np.all(np.isfinite(one))
    assert np.array_equal(one, run())


def test_workload_hgemm_splitk():
    """The 128 x 128 x 16384 product of one output tile, every output checked."""
    A, B = inputs.workload_operands("hgemm_nt_128x128x16384")
    got = gpu_f16_splitk(A, B)
    res = f16_check(got, oracle.gemm_f16_nt_exact(A, B),
                    oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))
    say("[hgemm_nt_128x128x16384] checked %d outputs, max %.2f ulp" % (res["count"],
                                                                       res["max_ulps"]))


# ---------------------------------------------- register-staged path ------
# Large products the full tiles cannot read in place (ragged M, N or K, rows
# at 2-byte offsets, odd leading dimensions, C unaligned): the wide-tile
# kernel with register-staged loads reads the operands where they are.  The
# K values reach every tail form of the last slab: whole slabs (640, 896),
# one element past a slab (1025), 9, 23 and 4 elements into the slab with the
# last chunk shifted by 7, 1 and 4 (777, 1111, 1100), K % 8 = 2, 3, 5, 6
# (1002, 1003, 1005, 1006), and a slab wholly past K when the slab count is
# rounded up to an even number (1025, 1111).  N = 3001 and 1000 exercise the
# 256 x 224 tiles as well as the 256 x 256 ones.  Rows at 16-byte addresses (K
# a multiple of 8 here) and K > 64 take the full tiles' ragged form instead
# when M and N are at least 128; the others with such rows take the direct
# copies, whose tail slabs are fixed in LDS: K below one slab (24: the first
# slab is the tail), M below 128 with 8 elements in the last slab (100 x
# 30000 x 1000).
STAGED_SHAPES = [(1000, 1001, 1111), (2048, 1000, 640), (1000, 2048, 640), (1024, 1024, 1025),
                 (1536, 1000, 777), (1111, 1152, 896), (1300, 1000, 1100), (1024, 1100, 1002),
                 (1100, 1024, 1003), (1024, 1024, 1005), (1050, 1030, 1006), (700, 3001, 600),
                 (1040, 1000, 1000), (1024, 1040, 1056), (6144, 7424, 24), (100, 30000, 1000)]


@pytest.mark.parametrize("shape", STAGED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f16_staged_shapes(shape, path_mode):
    M, N, K = shape
    A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
    got = gpu_f16(A, B, expect=expected_f16_path(path_mode, M, N, K))
    f16_check(got, oracle.gemm_f16_nt_exact(A, B), oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))


# Large products that are not whole tiles but whose rows start at 16-byte
# addresses (K % 8 == 0, at least 256 tiles of 256 x 256) run on the full-tile
# kernels' ragged form: the last tile row and column shifted back to end at M
# and N, the last slab's chunks past K zeroed in LDS.  Ragged M and N with 40
# K values in the last slab (4100 x 4200 x 1000), two slabs of which the
# second holds 8 (4000 x 4000 x 72), N ragged only and K whole slabs (4096 x
# 4104 x 2048: 256 x 224 tiles would need 2 rounds against 2 of 256 x 256),
# and bf16.  Every output against the oracle.
RAGGED16_SHAPES = [(4100, 4200, 1000), (4000, 4000, 72), (4096, 4104, 2048)]


@pytest.mark.parametrize("shape", RAGGED16_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f16_ragged_full_tiles(shape, path_mode):
    M, N, K = shape
    A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
    got = gpu_f16(A, B, expect=expected_f16_path(path_mode, M, N, K))
    f16_check(got, oracle.gemm_f16_nt_exact(A, B), oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))


def test_f16_ragged_full_tiles_c_unaligned_and_fused():
    """C one element into its buffer with an odd leading dimension (nothing
    outside C's window changes), then the fused write-back with the bias one
    element into its buffer (bf16 and the other layouts: test_layouts_gpu)."""
    M, N, K = 4100, 4100, 520
    A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
    bufC = torch.full((M * (N + 3) + 2,), 5.0, device=DEV, dtype=torch.float16)
    dC = bufC[1:1 + M * (N + 3)].view(M, N + 3)[:, :N]
    assert dg.f16_nt_path(dev(A), dev(B), dC) == "f16_mfma"
    dg.gemm_f16_nt(dev(A), dev(B), dC)
    torch.cuda.synchronize()
    f16_check(dC.cpu().numpy(), oracle.gemm_f16_nt_exact(A, B),
              oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))
    full = bufC.cpu().numpy()
    mask = np.ones(full.shape, bool)
    idx = 1 + np.arange(M)[:, None] * (N + 3) + np.arange(N)[None, :]
    mask[idx.ravel()] = False
    assert np.all(full[mask] == 5.0)
    A, B, bias, res = epi_operands(M, N, K, True, True)
    bbuf = torch.zeros(N + 1, device=DEV, dtype=torch.float16)
    bbuf[1:].copy_(dev(bias))
    dC = torch.full((M, N), float("nan"), device=DEV, dtype=torch.float16)
    assert dg.f16_nt_ex_path(dev(A), dev(B), dC, bbuf[1:], "silu", dev(res)) == "f16_mfma"
    dg.gemm_f16_nt_ex(dev(A), dev(B), dC, bbuf[1:], "silu", dev(res))
    torch.cuda.synchronize()
    check_ex(dC.cpu().numpy(), A, B, bias, "silu", res)


# Products with at most as many 64 x 64 tiles as CUs and K a multiple of 128
# run on the small-tile kernel that splits K across the four waves of a
# workgroup: 32 x 32 tiles (512 x 512 x 16384 and 1024 x 512 x 1024: 256 and
# 512 tiles), 16 x 16 tiles (256 x 256 x 8192, 512 x 256 x 4096), a short
# last chunk (2176 = 8 x 256 + 128).  Every output against the oracle, then
# bitwise repeats.
SMALL16_SHAPES = [(512, 512, 16384), (256, 256, 8192), (128, 512, 2176), (512, 256, 4096),
                  (1024, 512, 1024)]


@pytest.mark.parametrize("shape", SMALL16_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f16_small_tiles_split_k_in_workgroup(shape, path_mode):
    M, N, K = shape
    A, B = inputs.hgemm_nt_operands(M, N, K)
    got = gpu_f16(A, B, expect=expected_f16_path(path_mode, M, N, K))
    f16_check(got, oracle.gemm_f16_nt_exact(A, B), oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))
    assert np.array_equal(gpu_f16(A, B).view(np.uint16), got.view(np.uint16))


def test_f16_staged_small_integers_are_exact():
    """Small-integer operands make every partial sum exact, so the staged
    kernel (ragged M, N, K with a K tail) must equal the exact product
    rounded once, bit for bit; ties to even included."""
    M, N, K = 1030, 1040, 1027
    A = inputs.small_ints((M, K), 31, -2, 2, np.float16)
    B = inputs.small_ints((N, K), 32, -2, 2, np.float16)
    got = gpu_f16(A, B, expect="f16_staged")
    exact = A.astype(np.float64) @ B.astype(np.float64).T
    assert np.array_equal(got.view(np.uint16), oracle.half_from_double(exact).view(np.uint16))


def test_f16_staged_unaligned_and_c_only():
    """Operands one element into their buffers with odd leading dimensions
    (the register-staged wide tiles); then aligned operands with only C
    misaligned (the full tiles' ragged form, C at any 2-byte address).
    Nothing outside C's window changes."""
    for (M, N, K, off_ab) in [(1030, 1100, 1000, 1), (1024, 1024, 1024, 0)]:
        lda, ldb = (K + 3, K + 1) if off_ab else (K, K)
        ldc = N + 5
        A, B = inputs.hgemm_nt_operands(M, N, K, dist="normal")
        bufA = torch.zeros(M * lda + 8, device=DEV, dtype=torch.float16)
        bufB = torch.zeros(N * ldb + 8, device=DEV, dtype=torch.float16)
        bufC = torch.full((M * ldc + 2,), 5.0, device=DEV, dtype=torch.float16)
        dA = bufA[off_ab:off_ab + M * lda].view(M, lda)[:, :K]
        dB = bufB[off_ab:off_ab + N * ldb].view(N, ldb)[:, :K]
        dC = bufC[1:1 + M * ldc].view(M, ldc)[:, :N]
        dA.copy_(dev(A))
        dB.copy_(dev(B))
        assert dg.f16_nt_path(dA, dB, dC) == ("f16_staged" if off_ab else "f16_mfma")
        dg.gemm_f16_nt(dA, dB, dC)
        torch.cuda.synchronize()
        f16_check(dC.cpu().numpy(), oracle.gemm_f16_nt_exact(A, B),
                  oracle.gemm_f16_nt_exact(abs16(A), abs16(B)))
        full = bufC.cpu().numpy()
        mask = np.ones(full.shape, bool)
        idx = 1 + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
        mask[idx.ravel()] = False
        assert np.all(full[mask] == 5.0)


@pytest.mark.parametrize("act,use_bias,use_res", EPI_CASES)
def test_f16_staged_fused(act, use_bias, use_res):
    """The fused write-back on the staged path (a ragged shape with K odd),
    then on an aligned shape with the bias one element into its buffer and
    the residual rows of odd length, in place (the full tiles' ragged form)."""
    M, N, K = 1000, 1001, 1111
    A, B, bias, res = epi_operands(M, N, K, use_bias, use_res)
    dA, dB = dev(A), dev(B)
    dbias = dev(bias) if bias is not None else None
    dres = dev(res) if res is not None else None
    dC = torch.full((M, N), float("nan"), device=DEV, dtype=torch.float16)
    assert dg.f16_nt_ex_path(dA, dB, dC, dbias, act, dres) == "f16_staged"
    dg.gemm_f16_nt_ex(dA, dB, dC, dbias, act, dres)
    torch.cuda.synchronize()
    check_ex(dC.cpu().numpy(), A, B, bias, act, res)
    if not use_bias:
        return
    M, N, K = 1024, 1024, 1024
    A, B, bias, res = epi_operands(M, N, K, True, True)
    bbuf = torch.zeros(N + 1, device=DEV, dtype=torch.float16)
    bbuf[1:].copy_(dev(bias))
    cbuf = torch.zeros(M, N + 1, device=DEV, dtype=torch.float16)
    cbuf[:, :N].copy_(dev(res))
    dC = cbuf[:, :N]
    # aligned operands: the full tiles' ragged form (bias, residual and C at
    # any 2-byte address), the residual read in place of C
    assert dg.f16_nt_ex_path(dev(A), dev(B), dC, bbuf[1:], act, dC) == "f16_mfma"
    dg.gemm_f16_nt_ex(dev(A), dev(B), dC, bbuf[1:], act, dC)
    torch.cuda.synchronize()
    check_ex(dC.cpu().numpy(), A, B, bias, act, res)


# ------------------------------------------------------ 64-bit offsets -------
def test_offsets_beyond_4_gib():
    """Leading dimensions large enough that row offsets exceed 2^32 bytes."""
    M, N, K = 256, 256, 64
    lda = (1 << 24) + 8                                     # 256 rows * 32 MiB = 8 GiB
    A, B = inputs.hgemm_nt_operands(M, N, K)
    big = torch.empty(M, lda, device=DEV, dtype=torch.float16)
    big[:, :K].copy_(dev(A))
    dB = dev(B)
    dC = torch.empty(M, N, device=DEV, dtype=torch.float16)
    assert dg.f16_nt_path(big[:, :K], dB, dC) == "f16_mfma"
    dg.gemm_f16_nt(big[:, :K], dB, dC)
    torch.cuda.synchronize()
    ref = oracle.gemm_f16_nt_exact(A, B)
    sab = oracle.gemm_f16_nt_exact(abs16(A), abs16(B))
    f16_check(dC.cpu().numpy(), ref, sab)
    del big
    lda32 = (1 << 23) + 4
    A32, B32, _ = inputs.sgemm_operands(M, N, K)
    big = torch.empty(M, lda32, device=DEV)
    big[:, :K].copy_(dev(A32))
    dC = torch.empty(M, N, device=DEV)
    dg.gemm_f32(big[:, :K], dev(B32), dC)
    torch.cuda.synchronize()
    f32_check(dC.cpu().numpy(), oracle.gemm_f32(A32, B32), f32_tolerance(K, 1.0, 1.0))
    del big
    torch.cuda.empty_cache()


# ------------------------------------------------------ full-size workloads ---
def sample_points(M, N, tiles, seed=0, n_random=20000):
    """Whole rows, whole columns, whole tiles and random points of an M x N output."""
    rng = np.random.default_rng(seed)
    rows, cols = [], []
    for i in sorted({0, 1, M // 2 + 3, M - 1}):
        rows.append(np.full(N, i))
        cols.append(np.arange(N))
    for j in sorted({0, N // 3, N - 1}):
        rows.append(np.arange(M))
        cols.append(np.full(M, j))
    for (r0, r1, c0, c1) in tiles:
        rr, cc = np.meshgrid(np.arange(r0, r1), np.arange(c0, c1), indexing="ij")
        rows.append(rr.ravel())
        cols.append(cc.ravel())
    rows.append(rng.integers(0, M, n_random))
    cols.append(rng.integers(0, N, n_random))
    return np.concatenate(rows).astype(np.int32), np.concatenate(cols).astype(np.int32)


def tile_windows(M, N, tm, tn):
    last_m, last_n = ((M - 1) // tm) * tm, ((N - 1) // tn) * tn
    mid_m, mid_n = ((M // 2) // tm) * tm, ((N // 3) // tn) * tn
    return [(0, min(tm, M), 0, min(tn, N)), (last_m, M, last_n, N),
            (mid_m, min(mid_m + tm, M), mid_n, min(mid_n + tn, N))]


@pytest.mark.parametrize("name", ["sgemm_256", "sgemm_1024"])
def test_workload_sgemm_small_full(name):
    w = inputs.WORKLOADS[name]
    A, B, _ = inputs.workload_operands(name)
    got = gpu_f32(A, B, w["alpha"], 0.0, expect="f32_mfma")
    f32_check(got, oracle.gemm_f32(A, B), f32_tolerance(w["K"], np.abs(A).max(), np.abs(B).max()))


# The streaming fp32 kernel: M and N multiples of 128 with at least one 128 x 128
# tile per CU (256 on MI355X) and K a multiple of 64.  2048 x 2048 x 64: one
# slab per tile, one tile per CU; 2176 x 2048: 272 tiles, so some workgroups
# walk two tiles (the copy stream crosses a tile boundary); 4096 x 2048: two
# tiles each.  Sampled outputs: whole rows, columns and tiles, and random points.
STREAM_SHAPES = [(2048, 2048, 64), (2176, 2048, 192), (4096, 2048, 128), (2048, 2304, 320)]


@pytest.mark.parametrize("shape", STREAM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_stream_shapes(shape):
    M, N, K = shape
    A, B, _ = inputs.sgemm_operands(M, N, K)
    got = gpu_f32(A, B, expect="f32_mfma")
    rows, cols = sample_points(M, N, tile_windows(M, N, 128, 128), n_random=5000)
    ref = oracle.gemm_f32_points(A, B, rows, cols)
    f32_check(got[rows, cols], ref, f32_tolerance(K, 1.0, 1.0))


def test_f32_stream_alpha_beta_padded_and_exact():
    """alpha, beta and padded leading dimensions (16-byte loads of C, copies
    at a row stride that is not a power of two), then small integers, which
    make the fp32 result exact and independent of the summation order."""
    M, N, K = 2176, 2048, 128
    pad = 4
    Abig, Bbig, Cbig = inputs.sgemm_operands(M, N + pad, K + pad, with_c=True)
    A, B, C = Abig[:, :K], Bbig[:K, :N], Cbig[:, :N]
    dA, dB, dC = dev(Abig), dev(Bbig), dev(Cbig)
    dAv, dBv, dCv = dA[:, :K], dB[:K, :N], dC[:, :N]
    assert dg.f32_path(dAv, dBv, dCv, -0.5, 0.5) == "f32_mfma"
    dg.gemm_f32(dAv, dBv, dCv, -0.5, 0.5)
    torch.cuda.synchronize()
    got = dC.cpu().numpy()
    rows, cols = sample_points(M, N, tile_windows(M, N, 128, 128), n_random=5000)
    ref = oracle.gemm_f32_points(A, B, rows, cols, -0.5, 0.5, C)
    f32_check(got[:, :N][rows, cols], ref, f32_tolerance(K, 1.0, 1.0, -0.5, 0.5, 1.0))
    # the padding columns of C are untouched
    assert np.array_equal(got[:, N:], Cbig[:, N:])

    Ai = inputs.small_ints((M, 1024), 11, -3, 3, np.float32)
    Bi = inputs.small_ints((1024, N), 12, -3, 3, np.float32)
    goti = gpu_f32(Ai, Bi, expect="f32_mfma")
    rows, cols = sample_points(M, N, tile_windows(M, N, 128, 128), n_random=5000)
    assert np.array_equal(goti[rows, cols].astype(np.float64), oracle.gemm_f32_points(Ai, Bi, rows, cols))


# The 64 x 64 streaming kernel: M and N multiples of 64 with fewer 128 x 128
# tiles than CUs (or not multiples of 128), K a multiple of 64.  64^3: a
# stream of one slab; 64 x 128 x 128: two workgroups of two slabs; 192 x 64 x
# 320: odd slab counts; 1088 x 1024 x 192: 272 tiles, so some workgroups
# reduce two tiles in turn; 32768 x 64 x 64 and 16384 x 128 x 128: 512 tiles
# of one or two slabs, two per workgroup (a reduction barrier every slab or
# two).  Compared element by element with the oracle.
STREAM64_SHAPES = [(64, 64, 64), (64, 128, 128), (192, 64, 320), (1088, 1024, 192), (512, 768, 1024),
                   (32768, 64, 64), (16384, 128, 128)]


@pytest.mark.parametrize("shape", STREAM64_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_stream64_shapes(shape):
    M, N, K = shape
    A, B, _ = inputs.sgemm_operands(M, N, K)
    got = gpu_f32(A, B, expect="f32_mfma")
    f32_check(got, oracle.gemm_f32(A, B), f32_tolerance(K, 1.0, 1.0))


def test_f32_stream64_alpha_beta_padded_and_exact():
    M, N, K = 1088, 1024, 128
    pad = 4
    Abig, Bbig, Cbig = inputs.sgemm_operands(M, N + pad, K + pad, with_c=True)
    A, B, C = Abig[:, :K], Bbig[:K, :N], Cbig[:, :N]
    dA, dB, dC = dev(Abig), dev(Bbig), dev(Cbig)
    dAv, dBv, dCv = dA[:, :K], dB[:K, :N], dC[:, :N]
    assert dg.f32_path(dAv, dBv, dCv, 1.5, -0.75) == "f32_mfma"
    dg.gemm_f32(dAv, dBv, dCv, 1.5, -0.75)
    torch.cuda.synchronize()
    got = dC.cpu().numpy()
    ref = oracle.gemm_f32(A, B, 1.5, -0.75, C)
    f32_check(got[:, :N], ref, f32_tolerance(K, 1.0, 1.0, 1.5, -0.75, 1.0))
    assert np.array_equal(got[:, N:], Cbig[:, N:])
    Ai = inputs.small_ints((M, 640), 13, -3, 3, np.float32)
    Bi = inputs.small_ints((640, N), 14, -3, 3, np.float32)
    assert np.array_equal(gpu_f32(Ai, Bi, expect="f32_mfma").astype(np.float64), oracle.gemm_f32(Ai, Bi))


# Products with at most half as many 64 x 64 tiles as CUs (K a multiple of
# 64) run on the small-tile kernel whose four waves split each K chunk of up
# to 256 four ways, with 16 x 16 tiles while 32 x 32 ones would leave CUs
# idle: one chunk (256^3, 64^3), a short last chunk (320 = 256 + 64, 192,
# 1088), sixteen chunks (512 x 512 x 4096), long K (256 x 256 x 16384, 512 x
# 256 x 8192), a wide strip; the 32 x 32 tiles at 512 x 512 x 4096 and
# 256 x 1024 x 320 (256 tiles each) and between a quarter and half as many
# 64 x 64 tiles as CUs (512 x 1024 x 2048, 768 x 512 x 1088: 128 and 96
# tiles of 64 x 64), the 16 x 16 ones at the others.  Element by element
# against the oracle; the smallest of these shapes also appear in the
# stream64 list above, which the small-tile kernel now takes.
SMALL32_SHAPES = [(256, 256, 256), (64, 64, 64), (128, 512, 320), (512, 512, 4096),
                  (64, 1024, 192), (256, 128, 1088), (256, 1024, 320), (256, 256, 16384),
                  (512, 256, 8192), (512, 1024, 2048), (768, 512, 1088)]


@pytest.mark.parametrize("shape", SMALL32_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_small32_shapes(shape):
    M, N, K = shape
    A, B, _ = inputs.sgemm_operands(M, N, K)
    got = gpu_f32(A, B, expect="f32_mfma")
    f32_check(got, oracle.gemm_f32(A, B), f32_tolerance(K, 1.0, 1.0))


@pytest.mark.parametrize("shape", [(256, 320, 576), (512, 512, 576)], ids=["16x16", "32x32"])
def test_f32_small32_alpha_beta_nan_exact_and_repeats(shape):
    """alpha / beta with C read, beta = 0 with NaN in C, padded leading
    dimensions (the padding untouched), small integers exact, and bitwise
    repeats (the four partial tiles are added in a fixed order), on both tile
    sizes."""
    M, N, K = shape
    pad = 4
    Abig, Bbig, Cbig = inputs.sgemm_operands(M, N + pad, K + pad, with_c=True)
    A, B, C = Abig[:, :K], Bbig[:K, :N], Cbig[:, :N]
    dA, dB, dC = dev(Abig), dev(Bbig), dev(Cbig)
    dAv, dBv, dCv = dA[:, :K], dB[:K, :N], dC[:, :N]
    assert dg.f32_path(dAv, dBv, dCv, 1.5, -0.75) == "f32_mfma"
    dg.gemm_f32(dAv, dBv, dCv, 1.5, -0.75)
    torch.cuda.synchronize()
    got = dC.cpu().numpy()
    f32_check(got[:, :N], oracle.gemm_f32(A, B, 1.5, -0.75, C),
              f32_tolerance(K, 1.0, 1.0, 1.5, -0.75, 1.0))
    assert np.array_equal(got[:, N:], Cbig[:, N:])
    one = gpu_f32(A, B, 1.0, 0.0)                     # C prefilled with NaN
    assert np.all(np.isfinite(one))
    assert np.array_equal(gpu_f32(A, B, 1.0, 0.0), one)
    assert np.array_equal(gpu_f32(A, B, 2.0, 0.0), 2.0 * one)
    Ai = inputs.small_ints((M, 1024), 15, -3, 3, np.float32)
    Bi = inputs.small_ints((1024, N), 16, -3, 3, np.float32)
    assert np.array_equal(gpu_f32(Ai, Bi, expect="f32_mfma").astype(np.float64), oracle.gemm_f32(Ai, Bi))


# Large ragged or unaligned fp32 products run on the edge kernel, which reads
# the operands in place: 1030 x 1100 x 1000 (ragged M, N and K), 2048 x 2048 x
# 2000 (K not a multiple of 64: the 16-deep full tiles), 2000^3.  The masked
# stores leave C outside M x N untouched.
RAGGED32_SHAPES = [(1030, 1100, 1000), (2048, 2048, 2000), (2000, 2000, 2000)]


@pytest.mark.parametrize("shape", RAGGED32_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_ragged_large(shape):
    M, N, K = shape
    A, B, C = inputs.sgemm_operands(M, N, K, with_c=True)
    dA, dB = dev(A), dev(B)
    big = torch.full((M + 3, N + 5), 7.0, device=DEV)
    dC = big[1:1 + M, 2:2 + N]                 # C not 16-byte aligned, odd leading dimension
    dC.copy_(dev(C))
    assert dg.f32_path(dA, dB, dC, 0.75, 0.5) == "f32_general"
    dg.gemm_f32(dA, dB, dC, 0.75, 0.5)
    torch.cuda.synchronize()
    got = big.cpu().numpy()
    ref = oracle.gemm_f32(A, B, 0.75, 0.5, C)
    f32_check(got[1:1 + M, 2:2 + N], ref, f32_tolerance(K, 1.0, 1.0, 0.75, 0.5, 1.0))
    outside = np.ones(got.shape, bool)
    outside[1:1 + M, 2:2 + N] = False
    assert np.all(got[outside] == 7.0)


# Large ragged fp32 products with 16-byte aligned rows (K a multiple of 4,
# at least as many 128 x 128 tiles as CUs) run on the streaming kernel's
# ragged form: the last tile row and column shifted back to end at M and N,
# the last slab's chunks and rows past K zeroed in LDS.  Tails of 40 and 56
# (2000 x 2100 x 1000, 3000^3), K below one slab (36: the only slab is the
# tail), no tail (4000 x 4096 x 4096, ragged M only), and leading dimensions
# of 2052 for N = 2050, so that the shifted last column of tiles starts 8
# bytes past a 16-byte boundary; every output against the oracle, alpha /
# beta with C read, then beta = 0 over NaN, C outside M x N untouched.
STREAM_RAGGED32_SHAPES = [(2000, 2100, 1000), (3000, 3000, 3000), (2100, 2048, 36),
                          (4000, 4096, 4096)]


@pytest.mark.parametrize("shape", STREAM_RAGGED32_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_stream_ragged(shape):
    M, N, K = shape
    A, B, C = inputs.sgemm_operands(M, N, K, with_c=True)
    got = gpu_f32(A, B, 0.75, 0.5, C.copy(), expect="f32_general")
    ref = oracle.gemm_f32(A, B, 0.75, 0.5, C)
    f32_check(got, ref, f32_tolerance(K, 1.0, 1.0, 0.75, 0.5, 1.0))
    got0 = gpu_f32(A, B, 1.0, 0.0, expect="f32_general")     # C prefilled with NaN
    f32_check(got0, oracle.gemm_f32(A, B), f32_tolerance(K, 1.0, 1.0))


def test_f32_stream_ragged_padded_rows():
    M, N, K, ld = 2048, 2050, 1000, 2052
    A, B, C = inputs.sgemm_operands(M, N, K, with_c=True)
    bufB = torch.zeros(K, ld, device=DEV)
    dB = bufB[:, :N]
    dB.copy_(dev(B))
    bufC = torch.full((M, ld), 7.0, device=DEV)
    dC = bufC[:, :N]
    dC.copy_(dev(C))
    assert dg.f32_path(dev(A), dB, dC, 0.75, 0.5) == "f32_general"
    dg.gemm_f32(dev(A), dB, dC, 0.75, 0.5)
    torch.cuda.synchronize()
    got = bufC.cpu().numpy()
    f32_check(got[:, :N], oracle.gemm_f32(A, B, 0.75, 0.5, C),
              f32_tolerance(K, 1.0, 1.0, 0.75, 0.5, 1.0))
    assert np.all(got[:, N:] == 7.0)


def test_f32_unaligned_operand_and_c_exact():
    """A starting one float into its buffer, then aligned operands with an
    unaligned C; small integers make both results exact."""
    M, N, K = 1024, 1024, 1024
    A = inputs.small_ints((M, K), 21, -3, 3, np.float32)
    B = inputs.small_ints((K, N), 22, -3, 3, np.float32)
    ref = oracle.gemm_f32(A, B)
    bufA = torch.zeros(M * K + 1, device=DEV)
    dA = bufA[1:].view(M, K)
    dA.copy_(dev(A))
    dC = torch.full((M, N), float("nan"), device=DEV)
    assert dg.f32_path(dA, dev(B), dC) == "f32_general"
    dg.gemm_f32(dA, dev(B), dC)
    torch.cuda.synchronize()
    assert np.array_equal(dC.cpu().numpy().astype(np.float64), ref)
    bufC = torch.full((M * N + 1,), float("nan"), device=DEV)
    dC2 = bufC[1:].view(M, N)
    assert dg.f32_path(dev(A), dev(B), dC2) == "f32_general"
    dg.gemm_f32(dev(A), dev(B), dC2)
    torch.cuda.synchronize()
    assert np.array_equal(dC2.cpu().numpy().astype(np.float64), ref)
    assert np.isnan(bufC[0].item())


def test_f32_stream_fallback_k_not_a_multiple_of_64():
    """K % 64 != 0 keeps the register-staged 128 x 128 kernel."""
    M, N, K = 2048, 2048, 80
    A, B, _ = inputs.sgemm_operands(M, N, K)
    got = gpu_f32(A, B, expect="f32_mfma")
    rows, cols = sample_points(M, N, tile_windows(M, N, 128, 128), n_random=5000)
    f32_check(got[rows, cols], oracle.gemm_f32_points(A, B, rows, cols), f32_tolerance(K, 1.0, 1.0))


@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_workload_sgemm_4096(beta):
    """The 4096^3 SGEMM, every output against the oracle (C prefilled with NaN
    for beta = 0)."""
    K = 4096
    A, B, C = inputs.workload_operands("sgemm_4096")
    got = gpu_f32(A, B, 1.0, beta, C.copy() if beta else None, expect="f32_mfma")
    ref = oracle.gemm_f32(A, B, 1.0, beta, C)
    tol = f32_tolerance(K, np.abs(A).max(), np.abs(B).max(), 1.0, beta, np.abs(C).max())
    err = f32_check(got, ref, tol)
    say("[sgemm_4096 beta %g] checked all %d outputs, max err %.3e (bound %.3e)"
        % (beta, got.size, err, tol))


@pytest.mark.parametrize("name,path", [("hgemm_nt_5376x5376x2048", "f16_mfma"),
                                       ("hgemm_nt_5000x3001x1537", "f16_staged"),
                                       ("hgemm_nt_2048x2304x768", "f16_mfma")])
def test_workload_hgemm(name, path):
    """Every output of the workload against the oracle; the count of outputs
    outside the bare two-ulp rule (inside the fp32-accumulation floor) is
    printed beside the gated result."""
    A, B = inputs.workload_operands(name)
    got = gpu_f16(A, B, expect=path)
    ref = oracle.gemm_f16_nt_exact(A, B)
    sab = oracle.gemm_f16_nt_exact(abs16(A), abs16(B))
    res = f16_check(got, ref, sab)
    say("[%s] checked all %d outputs, max %.2f ulp, literal-2ulp violations %d"
        % (name, res["count"], res["max_ulps"], res["literal_2ulp_violations"]))
