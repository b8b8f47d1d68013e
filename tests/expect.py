"""The kernel each call is expected to run (the library's selection rules,
restated for the GPU tests)."""
from __future__ import annotations


def splitk_ranges(M, N, K, slab):
    """The library's automatic split count (1 = no split).  16-bit: tiles x
    ranges within 400 workgroups, ranges at least 256 deep, a power of two,
    at least two.  fp32: within 512 workgroups, at least 64 deep, at least
    three.  Tiles of 128 x 128, K at least 2048, at most 64 ranges."""
    tiles = -(-M // 128) * -(-N // 128)
    if K < 2048:
        return 1
    if slab == 64:
        s = min(400 // tiles, K // 256, 64)
        while s & (s - 1):
            s &= s - 1
        return s if s >= 2 else 1
    s = min(512 // tiles, K // 64, 64)
    return s if s >= 3 else 1


def splitk_auto(M, N, K, slab):
    return splitk_ranges(M, N, K, slab) > 1


def expected_f32_path(mode, M, N, K):
    """For contiguous, 16-byte aligned operands.  The plain calls never split
    K; what the full tiles cannot read in place runs on the edge kernel."""
    if mode == "general":
        return "f32_general"
    tiles = M % 64 == 0 and N % 64 == 0 and K % 16 == 0
    return "f32_mfma" if tiles else "f32_general"


def expected_f16_path(mode, M, N, K):
    if mode == "general":
        return "f16_general"
    if K == 0:
        return "f16_zero"
    if min(M, N) <= 8:
        return "f16_gemv"
    fast = K % 64 == 0 and ((M % 256 == 0 and (N % 256 == 0 or N % 224 == 0)) or
                            (M % 128 == 0 and (N % 128 == 0 or N % 192 == 0)))
    if fast:
        return "f16_mfma"
    large = M * N * K >= 1 << 30
    if large and ragged_fits(M, N, K):
        return "f16_mfma"
    # the register-staged wide tiles take large products (from 2^30
    # multiply-adds, K at least 8) that the full tiles cannot read in place
    return "f16_staged" if large and K >= 8 else "f16_general"


def ragged_fits(M, N, K):
    """The full tiles' ragged form (contiguous operands: rows of K elements):
    M, N >= 128, K > 64 with K % 8 == 0."""
    return M >= 128 and N >= 128 and K > 64 and K % 8 == 0


def expected_ex_path(M, N, K, op_a, op_b):
    """gemm_ex with the binding's workspace (contiguous, aligned operands)."""
    nt = op_a == "n" and op_b == "t"
    if K == 0:
        return "f16_zero"
    if min(M, N) <= 8:
        return "f16_gemv"
    if splitk_auto(M, N, K, 64):
        return "f16_splitk"
    large = M * N * K >= 1 << 30 and K >= 8
    if kmajor_in_place(M, N, K, op_a, op_b):
        return "f16_mfma"
    # NT in place, or the other layouts through 16-byte aligned transposed copies
    fast = K % 64 == 0 and ((M % 256 == 0 and (N % 256 == 0 or N % 224 == 0)) or
                            (M % 128 == 0 and (N % 128 == 0 or N % 192 == 0)))
    if fast:
        return "f16_mfma"
    if large and ragged_fits(M, N, K):
        return "f16_mfma"
    return "f16_staged" if large else "f16_general"


def tile_cost(shapes, M, N, cus=256, ragged=False):
    """The library's tile cost model: ceil(tiles / slots) x tile-time over the
    shapes given as (bm, bn, slots per CU, tile-time) -- whole tiles, or
    ceil(M / bm) x ceil(N / bn) tiles at least one tile wide and tall
    (ragged); None if none fits."""
    best = None
    for bm, bn, per_cu, tt in shapes:
        if (M < bm or N < bn) if ragged else (M % bm or N % bn):
            continue
        tiles = -(-M // bm) * -(-N // bn) if ragged else (M // bm) * (N // bn)
        if (bm, bn) == (128, 128) and tiles <= cus:
            tt = 128 * 128 * 8 // 5    # one tile per CU
        c = -(-tiles // (per_cu * cus)) * tt
        best = c if best is None or c < best else best
    return best


SMALL_TILES = [(128, 128, 2, 2 * 128 * 128 * 6 // 5), (128, 192, 1, 128 * 192 * 4 // 3)]
NT_TILES = [(256, 256, 1, 256 * 256), (256, 224, 1, 256 * 224)] + SMALL_TILES


def kmajor_in_place(M, N, K, op_a, op_b, c_aligned=True):
    """gemm_ex NN, TT and TN (contiguous operands at 16-byte addresses):
    tiles of 256 x 256 (NN, TT), 224 x 256 (NN) or 256 x 224 (TT, TN),
    128 x 128 or 128 x 192 read the K-major operands in place, with no
    workspace -- whole tiles with K % 64 == 0 (C aligned), or the ragged form
    for products of at least 2^30 multiply-adds at least 128 wide and tall
    (K > 64; K % 8 == 0 for NN and TT) -- unless the NT tiles on transposed
    copies cost less in the tile model (256 CUs)."""
    if K == 0 or (op_a, op_b) == ("n", "t"):
        return False
    whole_k = K % 64 == 0
    if not whole_k and (K < 64 or ((op_a, op_b) != ("t", "n") and K % 8)):
        return False
    # contiguous K-major operands: rows of M (A stored [K][M]) or N (B stored
    # [K][N]) elements, at 16-byte addresses only for multiples of 8
    if (op_a == "t" and M % 8) or (op_b == "n" and N % 8):
        return False
    big = (224, 256, 1, 224 * 256) if (op_a, op_b) == ("n", "n") else (256, 224, 1, 256 * 224)
    square = [(256, 256, 1, 256 * 256)] if (op_a, op_b) != ("t", "n") else []
    shapes = square + [big] + SMALL_TILES
    if whole_k:
        kc = tile_cost(shapes, M, N)
        if kc is not None:
            if not c_aligned:
                return False
            nc = tile_cost(NT_TILES, M, N)
            return nc is None or kc <= nc
    if M * N * K < (1 << 30):
        return False
    kc = tile_cost(shapes, M, N, ragged=True)
    if kc is None:
        return False
    if whole_k:
        nc = tile_cost(NT_TILES, M, N)
        if nc is not None:
            return kc <= nc
    if K % 8 == 0:
        nc = tile_cost(NT_TILES, M, N, ragged=True)
        if nc is not None:
            return kc <= nc
    return True
