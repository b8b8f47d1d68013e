"""GPU parity of gemm_ex: bf16 and fp16 in all four operand layouts, with and
without the fused write-back, against the CPU oracle.

Layout N/T follows the library: op "n" means A stored M x K and B stored
K x N, op "t" means A stored K x M and B stored N x K, so ("n", "t") is the
A * B^T product of gemm_f16_nt.  bfloat16 arrays travel as uint16 bit
patterns on the host (numpy has no bfloat16) and as torch.bfloat16 tensors on
the GPU.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from dense_gemm_sgemm_amd import inputs
from expect import expected_ex_path, kmajor_in_place
from tolerance import check16

torch = pytest.importorskip("torch")
import dense_gemm_sgemm_amd as dg  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LAYOUTS = [("n", "t"), ("n", "n"), ("t", "n"), ("t", "t")]


@pytest.fixture(autouse=True)
def _announce(request):
    print("\n[gpu case] %s" % request.node.nodeid, flush=True)
    sys.stdout.flush()
    yield


def to_dev(x: np.ndarray, fmt: str):
    x = np.ascontiguousarray(x)
    if fmt == "f16":
        return torch.from_numpy(x).to(DEV)
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)


def to_host(t, fmt: str) -> np.ndarray:
    if fmt == "f16":
        return t.cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def dtype_of(fmt: str):
    return torch.float16 if fmt == "f16" else torch.bfloat16


def stored_shapes(M, N, K, op_a, op_b):
    return ((M, K) if op_a == "n" else (K, M)), ((K, N) if op_b == "n" else (N, K))


def absval(x: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f16":
        return (x.view(np.uint16) & np.uint16(0x7FFF)).view(np.float16)
    return x & np.uint16(0x7FFF)


def reference(A, B, op_a, op_b, fmt, bias=None, act="none", res=None):
    """(fp64 value, fp64 sums of |a*b|) of the product from the oracle."""
    ref = oracle.gemm_ex_exact(A, B, op_a, op_b, bias, act, res, fmt)
    sab = oracle.gemm_ex_exact(absval(A, fmt), absval(B, fmt), op_a, op_b, fmt=fmt)
    return ref, sab


def run_ex(A, B, op_a, op_b, fmt, M, N, bias=None, act="none", res=None, expect=None):
    dA, dB = to_dev(A, fmt), to_dev(B, fmt)
    dbias = to_dev(bias, fmt) if bias is not None else None
    dres = to_dev(res, fmt) if res is not None else None
    dC = torch.full((M, N), float("nan"), device=DEV, dtype=dtype_of(fmt))
    if expect is not None:
        assert dg.ex_path(dA, dB, dC, op_a, op_b, dbias, act, dres) == expect
    dg.gemm_ex(dA, dB, dC, op_a, op_b, dbias, act, dres)
    torch.cuda.synchronize()
    return to_host(dC, fmt)


# Shapes reach each kernel: fast tiles 256 x 256, 256 x 224, 128 x 128 and 128 x 192 (in the
# other layouts on transposed copies), the edge kernel (ragged, odd K), the matrix-vector
# kernel both ways, split-K, and the register-staged wide tiles (1000 x 1001 x 1111, on the
# transposed copies in the other layouts).
SHAPES = [(256, 256, 64), (512, 448, 128), (128, 128, 192), (384, 576, 192), (133, 70, 45),
          (257, 255, 65), (1, 300, 777), (300, 3, 1000), (4, 129, 4100), (512, 512, 16384),
          (300, 200, 5000), (1000, 1001, 1111)]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: "".join(l))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_layouts(shape, layout, fmt):
    M, N, K = shape
    op_a, op_b = layout
    sa, sb = stored_shapes(M, N, K, op_a, op_b)
    A, B = inputs.operands16(sa, sb, fmt)
    got = run_ex(A, B, op_a, op_b, fmt, M, N, expect=expected_ex_path(M, N, K, op_a, op_b))
    ref, sab = reference(A, B, op_a, op_b, fmt)
    check16(got, ref, sab, fmt)


EPI_CASES = [("silu", True, True), ("relu", True, False), ("none", False, True)]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("layout", [("n", "t"), ("n", "n"), ("t", "n")], ids=lambda l: "".join(l))
@pytest.mark.parametrize("shape", [(256, 224, 64), (256, 384, 128), (133, 70, 45), (1, 300, 4096),
                                   (300, 200, 5000), (1000, 1001, 1111)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("act,use_bias,use_res", EPI_CASES)
def test_layouts_fused(shape, layout, fmt, act, use_bias, use_res):
    M, N, K = shape
    op_a, op_b = layout
    sa, sb = stored_shapes(M, N, K, op_a, op_b)
    A, B = inputs.operands16(sa, sb, fmt)
    rng = np.random.default_rng(43)
    bias = res = None
    if use_bias:
        b = rng.normal(0, 1.5, N)
        bias = b.astype(np.float16) if fmt == "f16" else inputs.bf16_bits(b)
    if use_res:
        r = rng.normal(0, 2.0, (M, N))
        res = r.astype(np.float16) if fmt == "f16" else inputs.bf16_bits(r)
    got = run_ex(A, B, op_a, op_b, fmt, M, N, bias, act, res)
    ref, sab = reference(A, B, op_a, op_b, fmt, bias, act, res)
    dec = oracle.half_to_double if fmt == "f16" else oracle.bf16_to_double
    babs = 0.0 if bias is None else np.abs(dec(bias))[None, :]
    rabs = 0.0 if res is None else np.abs(dec(res))
    check16(got, ref, sab, fmt, babs, rabs, fused=True)


# Large ragged products in the other layouts: the K-major operands are copied
# transposed (rows of round8(K)) and the register-staged wide tiles (K % 8 !=
# 0, or N below 128) or the full tiles' ragged form (K % 8 == 0) run on the
# copies -- ragged M and N at several residues of 8 (1030, 1100, 1001, 1023,
# 2049), K tails of 9, 23 and 4 elements and a slab wholly past K (777, 1111,
# 1100), a 256 x 224 tile choice (N = 3001), and an N of 9 for a K-major B.
STAGED_LAYOUT_SHAPES = [(1030, 1100, 1000), (1000, 1001, 1111), (1023, 2049, 777),
                        (2049, 1023, 1100), (700, 3001, 600), (1024 * 128, 9, 1024)]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("layout", LAYOUTS[1:], ids=lambda l: "".join(l))
@pytest.mark.parametrize("shape", STAGED_LAYOUT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_layouts_staged_on_copies(shape, layout, fmt):
    M, N, K = shape
    op_a, op_b = layout
    sa, sb = stored_shapes(M, N, K, op_a, op_b)
    A, B = inputs.operands16(sa, sb, fmt)
    dA, dB = to_dev(A, fmt), to_dev(B, fmt)
    dC = torch.full((M, N), float("nan"), device=DEV, dtype=dtype_of(fmt))
    assert dg.ex_path(dA, dB, dC, op_a, op_b) == expected_ex_path(M, N, K, op_a, op_b)
    assert dg.ex_workspace_bytes(dA, dB, dC, op_a, op_b) > 0
    dg.gemm_ex(dA, dB, dC, op_a, op_b)
    torch.cuda.synchronize()
    ref, sab = reference(A, B, op_a, op_b, fmt)
    check16(to_host(dC, fmt), ref, sab, fmt)


def test_layouts_staged_unaligned_exact_and_fused():
    """K-major operands one element into their buffers with odd leading
    dimensions (copied transposed, then the register-staged wide tiles), C
    unaligned; small-integer operands make every product exact
    (bit for bit against the exact sum rounded once).  Then the fused
    write-back on the same path."""
    for (op_a, op_b) in LAYOUTS[1:]:
        M, N, K = 1030, 1100, 1003
        sa, sb = stored_shapes(M, N, K, op_a, op_b)
        A = inputs.small_ints(sa, 51, -2, 2, np.float16)
        B = inputs.small_ints(sb, 52, -2, 2, np.float16)
        lda, ldb, ldc = sa[1] + 3, sb[1] + 1, N + 5
        bufA = torch.zeros(sa[0] * lda + 2, device=DEV, dtype=torch.float16)
        bufB = torch.zeros(sb[0] * ldb + 2, device=DEV, dtype=torch.float16)
        bufC = torch.full((M * ldc + 2,), 5.0, device=DEV, dtype=torch.float16)
        dA = bufA[1:1 + sa[0] * lda].view(sa[0], lda)[:, :sa[1]]
        dB = bufB[1:1 + sb[0] * ldb].view(sb[0], ldb)[:, :sb[1]]
        dC = bufC[1:1 + M * ldc].view(M, ldc)[:, :N]
        dA.copy_(to_dev(A, "f16"))
        dB.copy_(to_dev(B, "f16"))
        assert dg.ex_path(dA, dB, dC, op_a, op_b) == "f16_staged"
        dg.gemm_ex(dA, dB, dC, op_a, op_b)
        torch.cuda.synchronize()
        An, Bn = oracle.nt_operands(A, B, op_a, op_b)
        exact = An.astype(np.float64) @ Bn.astype(np.float64).T
        got = dC.contiguous().cpu().numpy()
        assert np.array_equal(got.view(np.uint16), oracle.half_from_double(exact).view(np.uint16))
        full = bufC.cpu().numpy()
        mask = np.ones(full.shape, bool)
        idx = 1 + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
        mask[idx.ravel()] = False
        assert np.all(full[mask] == 5.0)
    for (op_a, op_b) in LAYOUTS[1:]:
        M, N, K = 1000, 1001, 1111
        sa, sb = stored_shapes(M, N, K, op_a, op_b)
        A, B = inputs.operands16(sa, sb, "f16")
        rng = np.random.default_rng(44)
        bias = rng.normal(0, 1.5, N).astype(np.float16)
        res = rng.normal(0, 2.0, (M, N)).astype(np.float16)
        got = run_ex(A, B, op_a, op_b, "f16", M, N, bias, "silu", res, expect="f16_staged")
        ref, sab = reference(A, B, op_a, op_b, "f16", bias, "silu", res)
        check16(got, ref, sab, "f16", np.abs(bias.astype(np.float64))[None, :],
                np.abs(res.astype(np.float64)), fused=True)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_layouts_strided_unaligned_operands(fmt):
    """Stored operands one element into their buffers with padded rows, for
    every layout; C's padding is not written."""
    for (op_a, op_b) in LAYOUTS:
        for (M, N, K) in [(256, 256, 128), (133, 70, 45), (1, 200, 300)]:
            sa, sb = stored_shapes(M, N, K, op_a, op_b)
            A, B = inputs.operands16(sa, sb, fmt)
            lda, ldb, ldc = sa[1] + 3, sb[1] + 1, N + 5
            dt = dtype_of(fmt)
            bufA = torch.zeros(sa[0] * lda + 2, device=DEV, dtype=dt)
            bufB = torch.zeros(sb[0] * ldb + 2, device=DEV, dtype=dt)
            bufC = torch.full((M * ldc + 2,), 5.0, device=DEV, dtype=dt)
            dA = bufA[1:1 + sa[0] * lda].view(sa[0], lda)[:, :sa[1]]
            dB = bufB[1:1 + sb[0] * ldb].view(sb[0], ldb)[:, :sb[1]]
            dC = bufC[1:1 + M * ldc].view(M, ldc)[:, :N]
            dA.copy_(to_dev(A, fmt))
            dB.copy_(to_dev(B, fmt))
            dg.gemm_ex(dA, dB, dC, op_a, op_b)
            torch.cuda.synchronize()
            ref, sab = reference(A, B, op_a, op_b, fmt)
            check16(to_host(dC.contiguous(), fmt), ref, sab, fmt)
            full = to_host(bufC, fmt)
            mask = np.ones(full.shape, bool)
            idx = 1 + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]
            mask[idx.ravel()] = False
            five = np.float16(5.0) if fmt == "f16" else inputs.bf16_bits(np.array([5.0]))[0]
            assert np.all(full[mask] == five)


def test_bf16_exact_cases_and_determinism():
    """Small-integer bf16 products are exact below 256 and round ties to even
    above; repeated runs agree bitwise."""
    A = inputs.bf16_bits(inputs.small_ints((256, 128), 1, -1, 1, np.float64))
    B = inputs.bf16_bits(inputs.small_ints((256, 128), 2, -1, 1, np.float64))
    got = run_ex(A, B, "n", "t", "bf16", 256, 256)
    exact = oracle.bf16_to_double(A) @ oracle.bf16_to_double(B).T
    assert np.array_equal(got, oracle.bf16_from_double(exact))
    K = 576
    A = inputs.bf16_bits(np.ones((256, K)))
    B = np.zeros((256, K), np.uint16)
    for row, total in enumerate([257, 258, 259, 261, 255, 513]):
        B[row, :total] = inputs.bf16_bits(np.ones(total))
    got = run_ex(A, B, "n", "t", "bf16", 256, 256)
    assert list(oracle.bf16_to_double(got[0, :6])) == [256.0, 258.0, 260.0, 260.0, 255.0, 512.0]
    A, B = inputs.operands16((512, 256), (256, 256), "bf16")
    assert np.array_equal(run_ex(A, B, "n", "n", "bf16", 512, 256),
                          run_ex(A, B, "n", "n", "bf16", 512, 256))


@pytest.mark.parametrize("fmt,layout", [("bf16", ("n", "t")), ("f16", ("n", "n")),
                                        ("bf16", ("t", "n")), ("f16", ("t", "t"))])
def test_workload_5376_layouts(fmt, layout):
    """5376 x 5376 x 2048 in bf16 and in the other layouts, on the fast
    kernel, every output against the oracle."""
    M = N = 5376
    K = 2048
    op_a, op_b = layout
    sa, sb = stored_shapes(M, N, K, op_a, op_b)
    A, B = inputs.operands16(sa, sb, fmt, dist="uniform")
    got = run_ex(A, B, op_a, op_b, fmt, M, N, expect=expected_ex_path(M, N, K, op_a, op_b))
    An, Bn = oracle.nt_operands(A, B, op_a, op_b)
    ref = oracle.gemm_16_nt_exact(An, Bn, fmt)
    sab = oracle.gemm_16_nt_exact(absval(An, fmt), absval(Bn, fmt), fmt)
    r = check16(got, ref, sab, fmt)
    print("[5376^2 x 2048 %s %s] checked %d outputs, max %.2f ulp"
          % (fmt, "".join(layout), r["count"], r["max_ulps"]), flush=True)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K,op_a,op_b", [(1, 16384, 4096, "n", "n"), (2, 6000, 3001, "t", "n"),
                                             (8, 4096, 2048, "n", "n"), (5000, 1, 4099, "t", "t"),
                                             (3000, 6, 1024, "t", "n")])
def test_gemv_kmajor_weight(fmt, M, N, K, op_a, op_b):
    """Matrix-vector products whose long operand is stored K-major (B for
    op_b = "n", A for op_a = "t"): read in place, every output checked."""
    sa, sb = stored_shapes(M, N, K, op_a, op_b)
    A, B = inputs.operands16(sa, sb, fmt)
    got = run_ex(A, B, op_a, op_b, fmt, M, N, expect="f16_gemv")
    ref, sab = reference(A, B, op_a, op_b, fmt)
    r = check16(got, ref, sab, fmt)
    print("[gemv K-major %dx%dx%d %s%s %s] max %.2f ulp" % (M, N, K, op_a, op_b, fmt, r["max_ulps"]),
          flush=True)


# Large ragged products whose copies (or operands) have rows at 16-byte
# addresses run on the full-tile kernels' ragged form (K % 8 == 0, at least
# 256 tiles of 256 x 256): NT in place, NN and TN on the transposed copies,
# bf16 as well as fp16, with the fused write-back in NT.
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("layout", [("n", "t"), ("n", "n"), ("t", "n")], ids=lambda l: "".join(l))
def test_layouts_ragged_full_tiles(layout, fmt):
    M, N, K = 4100, 4104, 520
    op_a, op_b = layout
    sa, sb = stored_shapes(M, N, K, op_a, op_b)
    A, B = inputs.operands16(sa, sb, fmt)
    got = run_ex(A, B, op_a, op_b, fmt, M, N, expect="f16_mfma")
    ref, sab = reference(A, B, op_a, op_b, fmt)
    check16(got, ref, sab, fmt)
    if layout != ("n", "t"):
        return
    rng = np.random.default_rng(44)
    b = rng.normal(0, 1.5, N)
    r = rng.normal(0, 2.0, (M, N))
    bias = b.astype(np.float16) if fmt == "f16" else inputs.bf16_bits(b)
    res = r.astype(np.float16) if fmt == "f16" else inputs.bf16_bits(r)
    got = run_ex(A, B, op_a, op_b, fmt, M, N, bias, "silu", res, expect="f16_mfma")
    ref, sab = reference(A, B, op_a, op_b, fmt, bias, "silu", res)
    dec = oracle.half_to_double if fmt == "f16" else oracle.bf16_to_double
    check16(got, ref, sab, fmt, np.abs(dec(bias))[None, :], np.abs(dec(res)), fused=True)


# NN on whole 224 x 256 tiles, TT and TN on whole 256 x 224 tiles, all three
# on whole 128 x 128 or 128 x 192 tiles: the full-tile kernel reads the
# K-major operands in place (transposing LDS reads).  One
# tile with one slab, a few tiles, and more tiles than CUs (each workgroup
# then walks two tiles, prefetching across the tile boundary).
KMAJOR_CASES = [(("n", "n"), 224, 256, 64), (("n", "n"), 448, 512, 192),
                (("n", "n"), 672, 768, 320), (("n", "n"), 5376, 5376, 128),
                (("t", "t"), 256, 224, 64), (("t", "t"), 512, 448, 192),
                (("t", "t"), 768, 672, 320), (("t", "t"), 5376, 5376, 128),
                (("t", "n"), 256, 224, 64), (("t", "n"), 512, 448, 192),
                (("t", "n"), 768, 672, 320), (("t", "n"), 5376, 5376, 128),
                # 128 x 128 tiles (two workgroups per CU; 4096 x 3968: each walks
                # two tiles) and 128 x 192 tiles (one per CU; NN on the fused-QKV
                # shape)
                (("n", "n"), 384, 640, 192), (("t", "t"), 640, 384, 128),
                (("t", "n"), 384, 512, 256), (("n", "n"), 4096, 3968, 128),
                (("t", "n"), 4096, 3968, 64), (("n", "n"), 2048, 2304, 768),
                (("t", "t"), 256, 384, 192), (("t", "n"), 1024, 1152, 64),
                # 256 x 256 tiles (NN and TT; one set of B fragments)
                (("n", "n"), 4096, 4096, 64), (("t", "t"), 4096, 4096, 128),
                # ragged M or N (K % 64 == 0): the K-major tiles' ragged form
                # (the K-major operands' rows, M or N elements, at 16-byte addresses)
                (("n", "n"), 4100, 4200, 64), (("t", "t"), 5000, 3001, 128),
                (("t", "n"), 4104, 4112, 64), (("n", "n"), 5152, 5376, 64),
                (("t", "n"), 1000, 1104, 1024), (("t", "t"), 1104, 1030, 1024),
                # K not a multiple of 64: the ragged form's last slab copied
                # from K - 64, its repeated positions zeroed (TN: any K)
                (("n", "n"), 4100, 4200, 1000), (("t", "t"), 5000, 3001, 1000),
                (("t", "n"), 1000, 1104, 1001), (("n", "n"), 4096, 4096, 72),
                (("t", "n"), 4096, 4096, 100)]


def run_in_place(A, B, op_a, op_b, fmt, M, N, pad=0, bias=None, act="none", res=None):
    """gemm_ex with an empty workspace (the call fails if it needs one); the
    K-major operand optionally in rows padded by `pad` elements."""
    def stored(x, kmajor):
        if not (kmajor and pad):
            return to_dev(x, fmt)
        return to_dev(np.pad(x, ((0, 0), (0, pad))), fmt)[:, :x.shape[1]]
    dA = stored(A, op_a == "t")
    dB = stored(B, op_b == "n")
    dbias = to_dev(bias, fmt) if bias is not None else None
    dres = to_dev(res, fmt) if res is not None else None
    dC = torch.full((M, N), float("nan"), device=DEV, dtype=dtype_of(fmt))
    assert dg.ex_path(dA, dB, dC, op_a, op_b, dbias, act, dres) == "f16_mfma"
    dg.gemm_ex(dA, dB, dC, op_a, op_b, dbias, act, dres,
               workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    return to_host(dC, fmt)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("layout,M,N,K", KMAJOR_CASES,
                         ids=lambda v: "".join(v) if isinstance(v, tuple) else str(v))
def test_layouts_kmajor_in_place(layout, M, N, K, fmt):
    """Every output against the oracle, with no workspace; the larger
    shapes also with the K-major operand's rows padded by 8 elements."""
    op_a, op_b = layout
    assert kmajor_in_place(M, N, K, op_a, op_b)
    sa, sb = stored_shapes(M, N, K, op_a, op_b)
    A, B = inputs.operands16(sa, sb, fmt)
    ref, sab = reference(A, B, op_a, op_b, fmt)
    check16(run_in_place(A, B, op_a, op_b, fmt, M, N), ref, sab, fmt)
    if 448 * 512 <= M * N <= 4096 * 2048 or (M % 64 and N % 64):
        check16(run_in_place(A, B, op_a, op_b, fmt, M, N, pad=8), ref, sab, fmt)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("layout,M,N,K,act", [(("n", "n"), 448, 512, 192, "silu"),
                                              (("t", "t"), 512, 448, 256, "relu"),
                                              (("t", "n"), 512, 448, 128, "silu"),
                                              (("n", "n"), 4100, 4200, 64, "silu"),
                                              (("t", "t"), 4104, 4200, 1000, "relu")],
                         ids=lambda v: "".join(v) if isinstance(v, tuple) else str(v))
def test_layouts_kmajor_in_place_fused(layout, M, N, K, act, fmt):
    """The fused write-back (bias, activation, residual) on the in-place
    NN / TT kernels, against the oracle."""
    op_a, op_b = layout
    sa, sb = stored_shapes(M, N, K, op_a, op_b)
    A, B = inputs.operands16(sa, sb, fmt)
    rng = np.random.default_rng(45)
    b = rng.normal(0, 1.5, N)
    r = rng.normal(0, 2.0, (M, N))
    bias = b.astype(np.float16) if fmt == "f16" else inputs.bf16_bits(b)
    res = r.astype(np.float16) if fmt == "f16" else inputs.bf16_bits(r)
    got = run_in_place(A, B, op_a, op_b, fmt, M, N, bias=bias, act=act, res=res)
    ref, sab = reference(A, B, op_a, op_b, fmt, bias, act, res)
    dec = oracle.half_to_double if fmt == "f16" else oracle.bf16_to_double
    check16(got, ref, sab, fmt, np.abs(dec(bias))[None, :], np.abs(dec(res)), fused=True)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("M,N,K", [(1792, 1792, 192), (4096, 4096, 64)])
def test_kmajor_layouts_bitwise_equal_nt(fmt, M, N, K):
    """The in-place NN, TT and TN kernels take the same k order per output as
    the NT kernel (the same k bijection inside a k-step, the same slab
    order), so on the same values every layout gives the NT result bit for
    bit, in place or on copies; the NT result is itself checked against the
    oracle."""
    # 1792: whole tiles of 224 x 256 and 256 x 224; 4096: of 256 x 256
    A, Bt = inputs.operands16((M, K), (N, K), fmt)
    ref, sab = reference(A, Bt, "n", "t", fmt)
    nt = run_ex(A, Bt, "n", "t", fmt, M, N, expect="f16_mfma")
    check16(nt, ref, sab, fmt)
    stored = {"n": (np.ascontiguousarray(A), np.ascontiguousarray(Bt.T)),
              "t": (np.ascontiguousarray(A.T), np.ascontiguousarray(Bt))}
    for op_a, op_b in [("n", "n"), ("t", "t"), ("t", "n")]:
        sa = stored["n"][0] if op_a == "n" else stored["t"][0]
        sb = stored["n"][1] if op_b == "n" else stored["t"][1]
        # (TN 4096^2 runs on transposed copies, with the NT kernel)
        got = (run_in_place(sa, sb, op_a, op_b, fmt, M, N) if kmajor_in_place(M, N, K, op_a, op_b)
               else run_ex(sa, sb, op_a, op_b, fmt, M, N))
        assert np.array_equal(got.view(np.uint16), nt.view(np.uint16)), (op_a, op_b)
