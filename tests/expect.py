"""The kernel each call is expected to run (the library's selection rules,
restated for the GPU tests)."""
from __future__ import annotations


def splitk_auto(M, N, K, slab):
    """The library's split-K rule: K of at least 2048 and at least three ranges,
    with tiles x ranges within 512 workgroups (tiles of 128 x 128) and ranges
    at least 256 (fp16) or 64 (fp32) deep."""
    tiles = -(-M // 128) * -(-N // 128)
    if K < 2048:
        return False
    return min(512 // tiles, K // (256 if slab == 64 else 64), 64) >= 3


def expected_f32_path(mode, M, N, K):
    if mode == "general":
        return "f32_general"
    if splitk_auto(M, N, K, 16):
        return "f32_splitk"
    return "f32_mfma" if (M % 64 == 0 and N % 64 == 0 and K % 16 == 0) else "f32_general"


def expected_f16_path(mode, M, N, K):
    if mode == "general":
        return "f16_general"
    if K == 0:
        return "f16_zero"
    if min(M, N) <= 8:
        return "f16_gemv"
    if splitk_auto(M, N, K, 64):
        return "f16_splitk"
    fast = K % 64 == 0 and ((M % 256 == 0 and (N % 256 == 0 or N % 224 == 0)) or
                            (M % 128 == 0 and N % 128 == 0))
    return "f16_mfma" if fast else "f16_general"
