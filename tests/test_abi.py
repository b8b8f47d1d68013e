"""C-ABI checks that need no GPU: exported symbols, argument validation and
kernel selection.  None of these calls reaches the HIP runtime (validation
returns before the device check; the *_path functions are pure host code)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import dense_gemm_sgemm_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi355gemm.h")

F32_MFMA, F32_GENERAL, F32_SCALE = 3, 2, 1
F16_MFMA, F16_GENERAL, F16_ZERO, F16_GEMV = 6, 5, 4, 7
F16_SPLITK, F16_STAGED = 8, 10
ALIGNED = 0x100000          # fake device addresses: only their alignment is looked at
p = ctypes.c_void_p


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dg.LIB_PATH):
        from dense_gemm_sgemm_amd import build
        build.build()
    return dg.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MI355GEMM_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_symbols() == sorted(["gemm_f32", "gemm_f16_nt", "gemm_f16_nt_ex",
                                         "gemm_f32_splitk", "gemm_f16_nt_splitk",
                                         "gemm_f16_nt_splitk_static",
                                         "gemm_f32_splitk_workspace",
                                         "gemm_f16_nt_splitk_workspace", "gemm_ex",
                                         "gemm_ex_workspace",
                                         "gemm_ex_path",
                                         "gemm_status_string", "gemm_f32_path",
                                         "gemm_f16_nt_path", "gemm_f16_nt_ex_path",
                                         "gemm_path_name"])


def test_library_exports_exactly_the_header(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", dg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == declared_symbols()
    for name in declared_symbols():
        assert hasattr(lib, name)


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        s = dg.status_string(code)
        assert s and s != "unknown status code"
    assert dg.status_string(17) == "unknown status code"
    assert lib.gemm_path_name(3) == b"f32_mfma" and lib.gemm_path_name(99) == b"?"
    assert lib.gemm_path_name(F16_GEMV) == b"f16_gemv"
    assert lib.gemm_path_name(F16_STAGED) == b"f16_staged"


def f32(lib, M, N, K, alpha=1.0, A=ALIGNED, lda=None, B=ALIGNED, ldb=None, beta=0.0, C=ALIGNED,
        ldc=None):
    lda = max(1, K) if lda is None else lda
    ldb = max(1, N) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    return lib.gemm_f32_path(M, N, K, alpha, p(A) if A else None, lda, p(B) if B else None, ldb,
                             beta, p(C) if C else None, ldc)


def f16(lib, M, N, K, A=ALIGNED, lda=None, B=ALIGNED, ldb=None, C=ALIGNED, ldc=None):
    lda = max(1, K) if lda is None else lda
    ldb = max(1, K) if ldb is None else ldb
    ldc = max(1, N) if ldc is None else ldc
    return lib.gemm_f16_nt_path(M, N, K, p(A) if A else None, lda, p(B) if B else None, ldb,
                                p(C) if C else None, ldc)


def test_validation_codes(lib):
    assert f32(lib, -1, 4, 4) == -1 and f32(lib, 4, 4, -2) == -1 and f16(lib, 4, -1, 4) == -1
    assert f32(lib, 8, 8, 8, lda=7) == -2 and f32(lib, 8, 8, 8, ldb=7) == -2
    assert f32(lib, 8, 8, 8, ldc=7) == -2
    assert f16(lib, 8, 8, 8, lda=7) == -2 and f16(lib, 8, 8, 8, ldb=7) == -2
    assert f16(lib, 8, 8, 8, ldc=7) == -2
    assert f32(lib, 8, 8, 8, C=0) == -3 and f32(lib, 8, 8, 8, A=0) == -3
    assert f16(lib, 8, 8, 8, B=0) == -3 and f16(lib, 8, 8, 8, C=0) == -3
    # operands that are never read may be NULL
    assert f32(lib, 8, 8, 0, A=0, B=0) == F32_SCALE
    assert f32(lib, 8, 8, 8, alpha=0.0, A=0, B=0) == F32_SCALE
    assert f16(lib, 8, 8, 0, A=0, B=0) == F16_ZERO
    assert f32(lib, 0, 8, 8, A=0, B=0, C=0) == 0 and f16(lib, 8, 0, 8, A=0, B=0, C=0) == 0


def test_entry_points_reject_bad_arguments_before_any_device_call(lib):
    null = None
    assert lib.gemm_f32(-1, 1, 1, 1.0, null, 1, null, 1, 0.0, null, 1, null) == -1
    assert lib.gemm_f32(4, 4, 4, 1.0, p(ALIGNED), 4, p(ALIGNED), 3, 0.0, p(ALIGNED), 4, null) == -2
    assert lib.gemm_f16_nt(4, 4, 4, null, 4, p(ALIGNED), 4, p(ALIGNED), 4, null) == -3
    assert lib.gemm_f32(0, 5, 5, 1.0, null, 5, null, 5, 0.0, null, 5, null) == 0
    assert lib.gemm_f16_nt(5, 0, 5, null, 5, null, 5, null, 1, null) == 0


def f16ex(lib, M, N, K, A=ALIGNED, B=ALIGNED, bias=ALIGNED, act=0, res=ALIGNED, ldr=None,
          C=ALIGNED, ldc=None):
    ldr = max(1, N) if ldr is None else ldr
    ldc = max(1, N) if ldc is None else ldc
    return lib.gemm_f16_nt_ex_path(M, N, K, p(A) if A else None, max(1, K), p(B) if B else None,
                                   max(1, K), p(bias) if bias else None, act,
                                   p(res) if res else None, ldr, p(C) if C else None, ldc)


def test_fused_call_validation_and_paths(lib, monkeypatch):
    assert f16ex(lib, 8, 8, 8, act=3) == -6 and f16ex(lib, 8, 8, 8, act=-1) == -6
    assert f16ex(lib, 8, 8, 8, ldr=7) == -2
    assert f16ex(lib, 8, 8, 8, res=0, ldr=1) == F16_GEMV           # no residual: ldr unused
    assert f16ex(lib, 16, 16, 8, res=0, ldr=1) == F16_GENERAL
    assert f16ex(lib, 8, 8, 8, C=0) == -3 and f16ex(lib, 8, 8, 8, A=0) == -3
    assert f16ex(lib, 8, 8, 0, A=0, B=0) == F16_GENERAL              # K == 0: act(bias) + residual
    assert f16ex(lib, 0, 8, 8, A=0, B=0, C=0, act=3) == -6
    assert f16ex(lib, 0, 8, 8, A=0, B=0, C=0) == 0
    assert f16ex(lib, 5376, 5376, 2048) == F16_MFMA
    assert f16ex(lib, 5376, 5376, 2048, bias=0, res=0, act=2) == F16_MFMA
    # bias 2-byte aligned, residual rows unaligned: the full tiles' ragged form
    # (any alignment of C and the write-back operands), from 2^30
    # multiply-adds; rows of A or B at 2-byte addresses, K % 8 != 0, K <= 64
    # or M or N below 128: the register-staged wide tiles
    assert f16ex(lib, 5376, 5376, 2048, bias=ALIGNED + 2) == F16_MFMA
    assert f16ex(lib, 5376, 5376, 2048, ldr=5378) == F16_MFMA
    assert f16ex(lib, 2048, 4096, 2048, bias=ALIGNED + 2) == F16_MFMA
    assert f16ex(lib, 4100, 4200, 1000) == F16_MFMA                     # ragged, rows aligned
    assert f16ex(lib, 4100, 4200, 1001) == F16_STAGED                   # rows 2-byte aligned
    assert f16ex(lib, 3000, 3000, 3000) == F16_MFMA
    assert f16ex(lib, 100, 30000, 1000) == F16_STAGED                   # M < 128
    assert f16ex(lib, 256, 256, 64, bias=ALIGNED + 2) == F16_GENERAL     # too small
    assert f16ex(lib, 256, 224, 64, bias=ALIGNED + 2) == F16_GENERAL
    assert f16ex(lib, 5376, 5376, 2048, ldr=5380) == F16_MFMA
    assert f16ex(lib, 5000, 3001, 1537) == F16_STAGED
    assert f16ex(lib, 500, 301, 153) == F16_GENERAL                      # too small
    assert f16ex(lib, 1, 16384, 4096, bias=ALIGNED + 2, ldr=16385) == F16_GEMV  # any alignment
    assert f16ex(lib, 4096, 3, 4096, act=1) == F16_GEMV
    assert f16ex(lib, 1, 16384, 0, A=0, B=0) == F16_GENERAL
    monkeypatch.setenv("MI355GEMM_FORCE_PATH", "general")
    assert f16ex(lib, 5376, 5376, 2048) == F16_GENERAL
    null = None
    assert lib.gemm_f16_nt_ex(4, 4, 4, p(ALIGNED), 4, p(ALIGNED), 4, null, 7, null, 4, p(ALIGNED),
                              4, null) == -6


def test_path_selection(lib, monkeypatch):
    monkeypatch.delenv("MI355GEMM_FORCE_PATH", raising=False)
    assert f32(lib, 4096, 4096, 4096) == F32_MFMA
    assert f32(lib, 256, 256, 256) == F32_MFMA and f32(lib, 1024, 1024, 1024) == F32_MFMA
    assert f32(lib, 4096, 4096, 4096, beta=0.5) == F32_MFMA
    # ragged or unaligned fp32: the edge kernel reads the operands in place
    assert f32(lib, 4000, 4096, 4096) == F32_GENERAL                # ragged M
    assert f32(lib, 4032, 4096, 4096) == F32_MFMA                   # 64-row tiles
    assert f32(lib, 192, 320, 48) == F32_MFMA
    assert f32(lib, 4096, 4096, 4096, A=ALIGNED + 4) == F32_GENERAL  # 4-byte aligned only
    assert f32(lib, 4096, 4096, 4096, C=ALIGNED + 4) == F32_GENERAL
    assert f32(lib, 4096, 4096, 4000) == F32_MFMA                   # K % 16 == 0: 16-deep slabs
    assert f32(lib, 2000, 2000, 2000) == F32_GENERAL
    assert f32(lib, 1024, 1024, 1008) == F32_MFMA
    assert f32(lib, 1000, 1000, 1000) == F32_GENERAL
    assert f32(lib, 4096, 4096, 4096, lda=1 << 28) == F32_MFMA      # register-staged tiles
    assert f32(lib, 256, 256, 256, lda=258) == F32_GENERAL
    assert f16(lib, 5376, 5376, 2048) == F16_MFMA
    # ragged or unaligned and large: the full tiles' ragged form where A and
    # B rows start at 16-byte addresses (C anywhere) and there are 256 tiles
    # of 256 x 256, the register-staged wide tiles otherwise
    assert f16(lib, 5000, 3001, 1537) == F16_STAGED
    assert f16(lib, 5376, 5376, 2048, ldb=2052) == F16_STAGED
    assert f16(lib, 5376, 5376, 2048, C=ALIGNED + 8) == F16_MFMA
    assert f16(lib, 4096, 4104, 2048) == F16_MFMA and f16(lib, 6000, 6000, 64) == F16_STAGED  # K > 64
    assert f16(lib, 1500, 1500, 4096) == F16_MFMA and f16(lib, 1500, 1500, 4100) == F16_STAGED
    assert f16(lib, 1024, 1024, 1025) == F16_STAGED and f16(lib, 1024, 1024, 1000) == F16_GENERAL
    assert f16(lib, 1000, 1000, 1000) == F16_GENERAL                    # below 2^30 multiply-adds
    assert f16(lib, 128, 128, 64, C=ALIGNED + 2) == F16_GENERAL         # too small for wide tiles
    assert f16(lib, 1024, 1024, 1024, A=ALIGNED + 2, lda=1025) == F16_STAGED   # any alignment
    assert f16(lib, 1024, 1024, 7, A=ALIGNED + 2, lda=1025) == F16_GENERAL     # K < 8
    assert f16(lib, 1024, 1024, 1024, A=ALIGNED + 2, lda=(1 << 23) + 1) == F16_GENERAL  # offsets past 2^32
    assert f16(lib, 256, 224, 64) == F16_MFMA                       # 224-wide tiles
    assert f16(lib, 2048, 2304, 768) == F16_MFMA                    # 128 x 128 tiles
    assert f16(lib, 384, 640, 192) == F16_MFMA and f16(lib, 384, 640, 160) == F16_GENERAL
    assert f16(lib, 256, 256, 64, lda=(1 << 28) - 8) == F16_MFMA
    assert f16(lib, 256, 256, 64, lda=1 << 28) == F16_GENERAL         # 32-bit copy offsets
    # M or N at most 8: the matrix-vector kernel, whatever the alignment
    assert f16(lib, 1, 16384, 4096) == F16_GEMV and f16(lib, 16384, 1, 4096) == F16_GEMV
    assert f16(lib, 8, 16384, 4096) == F16_GEMV and f16(lib, 4096, 8, 4096) == F16_GEMV
    assert f16(lib, 1, 1, 1) == F16_GEMV and f16(lib, 3, 5, 7, A=ALIGNED + 2, lda=9) == F16_GEMV
    assert f16(lib, 9, 16384, 4096) != F16_GEMV and f16(lib, 16384, 9, 4096) != F16_GEMV
    assert f16(lib, 1, 16384, 0) == F16_ZERO
    monkeypatch.setenv("MI355GEMM_FORCE_PATH", "general")
    assert f16(lib, 1, 16384, 4096) == F16_GENERAL
    assert f32(lib, 4096, 4096, 4096) == F32_GENERAL
    assert f16(lib, 5376, 5376, 2048) == F16_GENERAL
    assert f32(lib, 8, 8, 0) == F32_SCALE


def test_split_k_plans(lib, monkeypatch):
    """The plain calls never split K (they need no workspace).  The explicit
    calls' automatic rule (splits <= 0) splits products with K >= 2048 and
    few 128 x 128 output tiles.  16-bit: tiles x ranges within 400
    workgroups, ranges at least 256 deep, a power of two, at least two.
    fp32: within 512 workgroups, at least 64 deep, at least three.  At most
    64 ranges, at most one per K slab; never for the matrix-vector shapes."""
    monkeypatch.delenv("MI355GEMM_FORCE_PATH", raising=False)
    assert f16(lib, 512, 512, 16384) == F16_MFMA and f16(lib, 128, 128, 16384) == F16_MFMA
    assert f16(lib, 300, 200, 5000) == F16_GENERAL
    assert f32(lib, 512, 512, 16384) == F32_MFMA and f32(lib, 100, 70, 3000) == F32_GENERAL
    ws16, ws32 = lib.gemm_f16_nt_splitk_workspace, lib.gemm_f32_splitk_workspace
    # 16 tiles -> 16 ranges of 16 slabs of 64
    assert ws16(512, 512, 16384, 0) == 16 * 512 * 512 * 4
    assert ws16(128, 128, 16384, 0) > 0 and ws16(1024, 1024, 4096, 0) > 0
    assert ws16(512, 512, 1024, 0) == 0                                # K below 2048
    assert ws16(2048, 2048, 8192, 0) == 0                              # 256 tiles
    assert ws16(1536, 1536, 4096, 0) == 2 * 1536 * 1536 * 4            # 144 tiles: 2 ranges
    assert ws16(1792, 1792, 4096, 0) == 2 * 1792 * 1792 * 4            # 196 tiles: 2 ranges
    assert ws16(2304, 2304, 4096, 0) == 0                              # 324 tiles: 1 range
    assert ws16(8, 512, 16384, 0) == 0                                 # the vector kernel
    assert ws16(1, 4096, 4096, 0) == 0
    assert ws16(100, 100, 1000, 3) == 3 * 128 * 128 * 4                # 16 slabs -> 6, 6, 4
    assert ws16(100, 100, 1000, 5) == 4 * 128 * 128 * 4                # 16 slabs -> 4 x 4
    assert ws16(64, 64, 100, 50) == 2 * 128 * 128 * 4                  # one range per slab
    assert ws16(64, 64, 100, 1) == 0 and ws16(0, 64, 100, 4) == 0 and ws16(64, 64, -1, 4) == 0
    assert ws16(300, 200, 5000, 0) == 16 * 384 * 256 * 4               # 5000 // 256 -> 16
    assert ws16(128, 128, 65536, 0) == 64 * 128 * 128 * 4              # at most 64 ranges
    assert ws32(512, 512, 16384, 0) == 32 * 512 * 512 * 4
    assert ws32(100, 70, 3000, 0) > 0 and ws32(4096, 4096, 4096, 0) == 0
    assert ws32(300, 257, 4099, 0) == 52 * 384 * 384 * 4               # 257 slabs / 56 -> 5 each
    assert ws32(130, 129, 40, 7) == 3 * 256 * 256 * 4                  # 3 slabs of 16
    monkeypatch.setenv("MI355GEMM_FORCE_PATH", "general")
    assert f16(lib, 512, 512, 16384) == F16_GENERAL and f32(lib, 512, 512, 16384) == F32_GENERAL


def ex(lib, type_, op_a, op_b, M, N, K, A=ALIGNED, lda=None, B=ALIGNED, ldb=None, bias=None,
       act=0, res=None, ldr=None, C=ALIGNED, ldc=None):
    lda = (max(1, K) if op_a == 0 else max(1, M)) if lda is None else lda
    ldb = (max(1, N) if op_b == 0 else max(1, K)) if ldb is None else ldb
    ldr = max(1, N) if ldr is None else ldr
    ldc = max(1, N) if ldc is None else ldc
    return lib.gemm_ex_path(type_, op_a, op_b, M, N, K, p(A) if A else None, lda,
                            p(B) if B else None, ldb, p(bias) if bias else None, act,
                            p(res) if res else None, ldr, p(C) if C else None, ldc)


def ex_ws(lib, type_, op_a, op_b, M, N, K, lda=None, ldb=None):
    lda = (max(1, K) if op_a == 0 else max(1, M)) if lda is None else lda
    ldb = (max(1, N) if op_b == 0 else max(1, K)) if ldb is None else ldb
    return lib.gemm_ex_workspace(type_, op_a, op_b, M, N, K, lda, ldb)


def test_gemm_ex_validation_and_paths(lib, monkeypatch):
    """Layouts: op N/T per operand with their leading-dimension rules; the
    other layouts run through transposed copies in the workspace, then on the
    A * B^T kernels the copies fit; unknown enumerations are
    GEMM_ERR_BAD_ARG."""
    monkeypatch.delenv("MI355GEMM_FORCE_PATH", raising=False)
    N_, T_ = 0, 1
    for t in (0, 1):
        assert ex(lib, t, N_, T_, 5376, 5376, 2048) == F16_MFMA
        assert ex(lib, t, N_, N_, 5376, 5376, 2048) == F16_MFMA      # B copied transposed
        assert ex(lib, t, T_, N_, 5376, 5376, 2048) == F16_MFMA
        assert ex(lib, t, T_, T_, 5376, 5376, 2048) == F16_MFMA
        assert ex(lib, t, T_, T_, 5000, 3001, 1537) == F16_STAGED    # ragged, on the copy
        assert ex(lib, t, T_, T_, 500, 301, 153) == F16_GENERAL      # through copies
        assert ex(lib, t, N_, N_, 1, 4096, 4096) == F16_GEMV
        assert ex(lib, t, T_, N_, 512, 512, 16384) == F16_SPLITK     # with its workspace
        # a copy has aligned, padded rows whatever the original alignment
        assert ex(lib, t, T_, T_, 256, 256, 64, A=ALIGNED + 2, lda=257) == F16_MFMA
        assert ex(lib, t, N_, T_, 256, 256, 64, A=ALIGNED + 2, lda=67) == F16_GENERAL
        assert ex(lib, t, T_, T_, 1024 * 1024, 9, 1024) == F16_STAGED
    # workspace sizes: none for NT and the plain vector kernel; the copies in
    # the other layouts; partial sums for K-major vectors
    assert ex_ws(lib, 0, N_, T_, 5376, 5376, 2048) == 0
    assert ex_ws(lib, 0, N_, N_, 5376, 5376, 2048) == 5376 * 2048 * 2
    assert ex_ws(lib, 0, N_, T_, 1, 4096, 4096) == 0
    assert ex_ws(lib, 0, T_, T_, 500, 301, 153) == (500 * 160 * 2 + 255) // 256 * 256
    assert ex_ws(lib, 0, N_, N_, 100, 300, 153) == 300 * 160 * 2
    assert ex_ws(lib, 0, N_, N_, 1, 16384, 4096) > 0                  # K-major weight
    assert ex_ws(lib, 0, N_, T_, 512, 512, 16384) == 16 * 512 * 512 * 4   # split-K partials
    assert ex_ws(lib, 0, N_, N_, 512, 512, 16384) == 512 * 16384 * 2 + 16 * 512 * 512 * 4
    assert ex_ws(lib, 0, N_, T_, -1, 5, 5) == 0 and ex_ws(lib, 7, N_, T_, 5, 5, 5) == 0
    assert ex(lib, 2, 0, 1, 8, 8, 8) == -6 and ex(lib, 0, 2, 1, 8, 8, 8) == -6
    assert ex(lib, 0, 0, -1, 8, 8, 8) == -6 and ex(lib, 0, 0, 1, 8, 8, 8, act=5) == -6
    # leading dimensions follow the stored shapes
    assert ex(lib, 0, T_, T_, 100, 8, 50, lda=99) == -2 and ex(lib, 0, T_, T_, 100, 8, 50) == F16_GEMV
    assert ex(lib, 0, N_, N_, 16, 100, 50, ldb=99) == -2 and ex(lib, 0, N_, N_, 16, 100, 50) > 0
    assert ex(lib, 0, N_, T_, 16, 16, 0, A=0, B=0) == F16_ZERO
    assert ex(lib, 0, N_, T_, 16, 16, 0, A=0, B=0, bias=ALIGNED) == F16_GENERAL
    assert ex(lib, 1, N_, T_, 0, 16, 5, A=0, B=0, C=0) == 0
    monkeypatch.setenv("MI355GEMM_FORCE_PATH", "general")
    assert ex(lib, 1, N_, N_, 5376, 5376, 2048) == F16_GENERAL
    null = None
    a = p(ALIGNED)
    assert lib.gemm_ex(3, 0, 1, 4, 4, 4, a, 4, a, 4, null, 0, null, 4, a, 4, null, 0, null) == -6
    monkeypatch.delenv("MI355GEMM_FORCE_PATH", raising=False)
    # a workspace the call needs is checked before any work: missing, too
    # small or misaligned
    need = ex_ws(lib, 0, T_, T_, 500, 301, 153)
    assert lib.gemm_ex(0, T_, T_, 500, 301, 153, a, 500, a, 153, null, 0, null, 0, a, 301, null,
                       0, null) == -7
    assert lib.gemm_ex(0, T_, T_, 500, 301, 153, a, 500, a, 153, null, 0, null, 0, a, 301, a,
                       need - 1, null) == -7
    assert lib.gemm_ex(0, T_, T_, 500, 301, 153, a, 500, a, 153, null, 0, null, 0, a, 301,
                       p(ALIGNED + 8), need, null) == -7


def test_gemm_ex_kmajor_in_place_needs_no_workspace(lib, monkeypatch):
    """NN on whole 224 x 256 tiles, TT and TN on whole 256 x 224 tiles read
    the K-major operands in place: a call without a workspace passes the
    workspace check and reaches the device check (no device here), where
    the copy paths stop at GEMM_ERR_WORKSPACE.  gemm_ex_workspace stays an
    upper bound for any pointers (the copies)."""
    monkeypatch.delenv("MI355GEMM_FORCE_PATH", raising=False)
    N_, T_ = 0, 1
    null = None
    a = p(ALIGNED)

    def call(op_a, op_b, M, N, K, A=a, lda=None, B=a, ldb=None):
        lda = (K if op_a == N_ else M) if lda is None else lda
        ldb = (N if op_b == N_ else K) if ldb is None else ldb
        return lib.gemm_ex(0, op_a, op_b, M, N, K, A, lda, B, ldb, null, 0, null, 0, a, N, null,
                           0, null)

    for op in ((N_, N_), (T_, T_)):
        assert call(*op, 5376, 5376, 2048) == -4
        assert ex_ws(lib, 0, *op, 5376, 5376, 2048) == 5376 * 2048 * 2
    assert call(T_, N_, 5376, 5376, 2048) == -4                     # TN: both in place
    assert ex_ws(lib, 0, T_, N_, 5376, 5376, 2048) == 2 * 5376 * 2048 * 2
    assert call(N_, N_, 448, 512, 64) == -4 and call(T_, T_, 512, 448, 64) == -4
    assert call(T_, N_, 512, 448, 64) == -4
    assert call(N_, T_, 5376, 5376, 2048) == -4                     # NT: always in place
    assert call(T_, N_, 5376, 5376 - 224, 2048) == -4
    # ragged M or N with K % 64 == 0: the K-major tiles' ragged form, in place
    assert call(T_, N_, 5376 - 224, 5376, 2048) == -4
    assert call(T_, T_, 5376 - 224, 5376, 2048) == -4
    assert call(N_, N_, 5376, 5000, 2048) == -4 and call(N_, N_, 4100, 4200, 1024) == -4
    assert call(N_, N_, 1000, 1000, 512) == -7                      # small: the copy
    assert call(N_, N_, 4100, 100, 4096) == -7                      # not 128 wide
    # 256 x 256 (NN, TT) and 128-row tiles in place; NN 4096 x 3584 goes
    # through the copy, where NT's 256 x 224 tiles take fewer tile-times than
    # NN's shapes, and so does TN 4096^2 (its K-major tiles stop at 256 x 224)
    assert call(N_, N_, 2048, 2304, 768) == -4 and call(T_, N_, 384, 512, 256) == -4
    assert call(T_, T_, 640, 384, 128) == -4
    for op in ((N_, N_), (T_, T_), (T_, N_)):
        assert call(*op, 4096, 3968, 128) == -4
    assert call(N_, N_, 4096, 4096, 4096) == -4 and call(T_, T_, 4096, 4096, 4096) == -4
    assert call(T_, N_, 4096, 4096, 4096) == -7                     # TN: no 256 x 256
    assert call(N_, N_, 4096, 3584, 128) == -7 and call(T_, T_, 4096, 3584, 128) == -4
    # K % 64 != 0: the ragged form's last slab copied from K - 64; NN and TT
    # need K % 8 == 0 (their K-contiguous operand), TN takes any K > 64
    assert call(N_, N_, 5376, 5376, 2000) == -4 and call(T_, T_, 4096, 4096, 1000) == -4
    assert call(T_, N_, 5376, 5376, 2001) == -4 and call(T_, N_, 4104, 4112, 1537) == -4
    assert call(N_, N_, 5376, 5376, 2001) == -7                     # A rows unaligned
    assert call(T_, N_, 2048, 2048, 40) == -7                       # small, K < 64
    assert call(N_, N_, 5376, 5376, 2048, B=p(ALIGNED + 2)) == -7   # B unaligned
    assert call(N_, N_, 5376, 5376, 2048, ldb=5380) == -7           # ldb % 8 != 0
    assert ex(lib, 0, N_, N_, 448, 512, 64) == F16_MFMA
    assert ex(lib, 0, T_, T_, 512, 448, 64) == F16_MFMA
    assert ex(lib, 0, T_, N_, 512, 448, 64) == F16_MFMA


def test_split_k_workspace_errors_need_no_device(lib):
    null = None
    a = p(ALIGNED)
    assert lib.gemm_f16_nt_splitk(512, 512, 16384, a, 16384, a, 16384, a, 512, 0, null, 0,
                                  null) == -7
    need = lib.gemm_f16_nt_splitk_workspace(512, 512, 16384, 0)
    assert lib.gemm_f16_nt_splitk(512, 512, 16384, a, 16384, a, 16384, a, 512, 0, a, need - 1,
                                  null) == -7
    assert lib.gemm_f16_nt_splitk(512, 512, 16384, a, 16384, a, 16384, a, 512, 0,
                                  p(ALIGNED + 8), need, null) == -7
    assert lib.gemm_f32_splitk(256, 256, 4096, 1.0, a, 4096, a, 256, 0.0, a, 256, 4, null, 0,
                               null) == -7
    assert lib.gemm_f32_splitk(-1, 256, 4096, 1.0, a, 4096, a, 256, 0.0, a, 256, 4, null, 0,
                               null) == -1
    assert lib.gemm_f16_nt_splitk(0, 5, 5, null, 5, null, 5, null, 5, 4, null, 0, null) == 0


def test_static_scratch_split_k_errors_need_no_device(lib):
    """gemm_f16_nt_splitk_static refuses, before any HIP call, a split whose
    partial sums exceed the static scratch area, and validates like the
    workspace call."""
    null = None
    a = p(ALIGNED)
    assert dg.STATIC_SCRATCH_BYTES == 32 << 20
    assert lib.gemm_f16_nt_splitk_workspace(1024, 1024, 16384, 16) > dg.STATIC_SCRATCH_BYTES
    assert lib.gemm_f16_nt_splitk_static(1024, 1024, 16384, a, 16384, a, 16384, a, 1024, 16,
                                         null) == dg.GEMM_ERR_SCRATCH_LIMIT
    assert lib.gemm_f16_nt_splitk_static(-1, 5, 5, a, 5, a, 5, a, 5, 0, null) == -1
    assert lib.gemm_f16_nt_splitk_static(5, 5, 5, a, 4, a, 5, a, 5, 0, null) == -2
    assert lib.gemm_f16_nt_splitk_static(5, 5, 5, null, 5, a, 5, a, 5, 0, null) == -3
    assert lib.gemm_f16_nt_splitk_static(0, 5, 5, null, 5, null, 5, null, 5, 4, null) == 0
    assert "static scratch" in dg.status_string(dg.GEMM_ERR_SCRATCH_LIMIT)


def test_python_binding_validates_tensors(lib):
    torch = pytest.importorskip("torch")
    a = torch.zeros(4, 4)
    with pytest.raises(TypeError):
        dg.gemm_f32(a, a, a)                       # CPU tensors are refused
    with pytest.raises(TypeError):
        dg.gemm_f16_nt(a, a, a)
