"""A seeded random sweep over gemm_ex's other layouts (NN, TT, TN): shapes
drawn as whole tiles of each in-place tile shape (256 x 256, 224 x 256,
256 x 224, 128 x 128, 128 x 192) and, one in four, near misses that are not
whole tiles; the K-major operand's rows padded by 0 or 8 elements (read in
place) or by 1 (rows off 16-byte addresses: the transposed copies).  fp16 or
bf16; every output compared with the oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from dense_gemm_sgemm_amd import inputs
from expect import kmajor_in_place
from tolerance import check16

torch = pytest.importorskip("torch")
import dense_gemm_sgemm_amd as dg  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
LAYOUTS = [("n", "n"), ("t", "t"), ("t", "n")]
TILES = {("n", "n"): [(256, 256), (224, 256), (128, 128), (128, 192)],
         ("t", "t"): [(256, 256), (256, 224), (128, 128), (128, 192)],
         ("t", "n"): [(256, 224), (128, 128), (128, 192)]}


def draw(seed):
    rng = np.random.default_rng(7000 + seed)
    op = LAYOUTS[int(rng.integers(0, 3))]
    fmt = "f16" if rng.integers(0, 2) == 0 else "bf16"
    bm, bn = TILES[op][int(rng.integers(0, len(TILES[op])))]
    while True:
        M, N = bm * int(rng.integers(1, 13)), bn * int(rng.integers(1, 13))
        K = 64 * int(rng.integers(1, 25))
        if rng.integers(0, 4) == 0:       # a near miss: not whole tiles, or a K tail
            which = int(rng.integers(0, 3))
            M, N, K = (M + 8 if which == 0 else M), (N + 8 if which == 1 else N), \
                (K + 8 if which == 2 else K)
        if M * N * K <= (1 << 30):
            break
    pad = int(rng.choice([0, 8, 1]))
    return op, fmt, M, N, K, pad


def to_dev(x: np.ndarray, fmt: str, pad: int):
    """A stored operand on the GPU, rows padded by `pad` elements."""
    x = np.ascontiguousarray(np.pad(x, ((0, 0), (0, pad))))
    t = torch.from_numpy(x if fmt == "f16" else x.view(np.int16)).to(DEV)
    if fmt == "bf16":
        t = t.view(torch.bfloat16)
    return t[:, :x.shape[1] - pad]


def absval(x: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "f16":
        return (x.view(np.uint16) & np.uint16(0x7FFF)).view(np.float16)
    return x & np.uint16(0x7FFF)


@pytest.mark.parametrize("seed", list(range(24)))
def test_random_layout_sweep(seed):
    (op_a, op_b), fmt, M, N, K, pad = draw(seed)
    print("\n[layout sweep] seed %d %s%s %s %dx%dx%d pad %d" % (seed, op_a, op_b, fmt, M, N, K, pad),
          flush=True)
    sys.stdout.flush()
    sa = (M, K) if op_a == "n" else (K, M)
    sb = (K, N) if op_b == "n" else (N, K)
    A, B = inputs.operands16(sa, sb, fmt)
    # the K-major operands' rows padded (the other one's rows stay packed)
    dA = to_dev(A, fmt, pad if op_a == "t" else 0)
    dB = to_dev(B, fmt, pad if op_b == "n" else 0)
    dC = torch.full((M, N), float("nan"), device=DEV,
                    dtype=torch.float16 if fmt == "f16" else torch.bfloat16)
    path = dg.ex_path(dA, dB, dC, op_a, op_b)
    in_place = pad != 1 and kmajor_in_place(M, N, K, op_a, op_b)
    if in_place:
        # an empty workspace: the call must not need one
        dg.gemm_ex(dA, dB, dC, op_a, op_b, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    else:
        dg.gemm_ex(dA, dB, dC, op_a, op_b)
    torch.cuda.synchronize()
    got = dC.cpu().numpy() if fmt == "f16" else dC.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.gemm_ex_exact(A, B, op_a, op_b, fmt=fmt)
    sab = oracle.gemm_ex_exact(absval(A, fmt), absval(B, fmt), op_a, op_b, fmt=fmt)
    r = check16(got, ref, sab, fmt)
    print("[layout sweep] seed %d path %s%s ok, max %.2f ulp"
          % (seed, path, " (in place)" if in_place else "", r["max_ulps"]), flush=True)
