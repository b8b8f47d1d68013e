"""Acceptance rules for GPU results against the oracle (host logic, no GPU).

fp32: max |C - Cref| <= 1e-5 * (|alpha| * K * max|A| * max|B| + |beta| * max|C_in|).
  With alpha = 1 and beta = 0 this is the bound 1e-5 * K * max|a| * max|b|; the
  beta term only adds the (tiny) rounding allowance of the beta * C_in summand.
fp16: |C - half(Cref)| <= 2 ulp16(half(Cref)) + 2^-23 * sum_k |A_ik B_jk|.
  ulp16(x) = 2^(max(floor(log2|x|), -14) - 10), the binary16 spacing at x.
  The second term is the fp32-accumulation floor that matters only near zero,
  where two half ulps are smaller than any fp32 sum's rounding error.
bf16: the same rules with the bfloat16 spacing (8 significant bits, normal
  exponents from -126) in place of binary16's.
fp16 with the fused write-back act(A B^T + bias) + residual: the same 2-ulp
  rule around the oracle's rounded value, with the floor widened to
  2^-22 * (sum |A_ik B_jk| + |bias_j| + |residual_ij| + |Cref|): the fp32
  additions of bias and residual, the activation's slope (at most 1.1 for
  SiLU) and its fp32 evaluation each add at most a few fp32 roundings.
"""
from __future__ import annotations

import numpy as np

import oracle


def f32_tolerance(K: int, amax: float, bmax: float, alpha: float = 1.0, beta: float = 0.0,
                  cmax: float = 0.0) -> float:
    return 1e-5 * (abs(alpha) * max(K, 1) * amax * bmax + abs(beta) * cmax)


def f32_check(got: np.ndarray, ref: np.ndarray, tol: float) -> float:
    """Returns the max abs error; raises AssertionError beyond ``tol``."""
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite values in the GPU result"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    assert err <= tol, "max |C - Cref| = %.3e exceeds %.3e" % (err, tol)
    return err


def ulp16(h: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(h, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -14.0)
    return np.where(a > 0, np.exp2(e - 10.0), 2.0 ** -24)


def f16_violations(got16: np.ndarray, ref: np.ndarray, sab: np.ndarray) -> dict:
    """Counts elements of ``got16`` outside the fp16 acceptance rule.

    ``ref`` is the oracle's fp64 sum, ``sab`` the sum of |a*b| for the same
    outputs.  Returns counts for the gated rule and for the bare 2-ulp rule."""
    ref16 = oracle.half_from_double(ref).astype(np.float64)
    g = np.asarray(got16, dtype=np.float64)
    diff = np.abs(g - ref16)
    two_ulp = 2.0 * ulp16(ref16)
    bad = ~(diff <= two_ulp + 2.0 ** -23 * sab)            # NaN counts as a violation
    literal = ~(diff <= two_ulp)
    with np.errstate(invalid="ignore", divide="ignore"):
        worst = float(np.nanmax(diff / ulp16(ref16))) if g.size else 0.0
    return {"violations": int(bad.sum()), "literal_2ulp_violations": int(literal.sum()),
            "max_ulps": worst, "count": int(g.size)}


def f16_check(got16: np.ndarray, ref: np.ndarray, sab: np.ndarray) -> dict:
    res = f16_violations(got16, ref, sab)
    assert res["violations"] == 0, "fp16 tolerance violated: %s" % res
    return res


def f16_ex_check(got16: np.ndarray, ref: np.ndarray, sab: np.ndarray, bias_abs=0.0,
                 res_abs=0.0) -> dict:
    """The fused write-back rule; ``ref`` is the oracle's fp64 value of
    act(A B^T + bias) + residual, ``sab`` the sums of |a*b|."""
    ref16 = oracle.half_from_double(ref).astype(np.float64)
    g = np.asarray(got16, dtype=np.float64)
    diff = np.abs(g - ref16)
    floor = 2.0 ** -22 * (sab + bias_abs + res_abs + np.abs(ref))
    bad = ~(diff <= 2.0 * ulp16(ref16) + floor)
    with np.errstate(invalid="ignore", divide="ignore"):
        worst = float(np.nanmax(diff / ulp16(ref16))) if g.size else 0.0
    res = {"violations": int(bad.sum()), "max_ulps": worst, "count": int(g.size)}
    assert res["violations"] == 0, "fused fp16 tolerance violated: %s" % res
    return res


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(a > 0, np.exp2(e - 7.0), 2.0 ** -133)


def check16(got, ref: np.ndarray, sab: np.ndarray, fmt: str = "f16", bias_abs=0.0,
            res_abs=0.0, fused: bool = False) -> dict:
    """The fp16 / bf16 acceptance rules.  ``got``: float16 values, or bfloat16
    bit patterns (uint16) when fmt is "bf16"; ``ref``: the oracle's fp64 value;
    ``sab``: the sums of |a*b|; ``fused``: the fused write-back's wider floor."""
    if fmt == "f16":
        ref16 = oracle.half_from_double(ref).astype(np.float64)
        g = np.asarray(got, dtype=np.float64)
        ulp = ulp16(ref16)
    else:
        ref16 = oracle.bf16_to_double(oracle.bf16_from_double(ref))
        g = oracle.bf16_to_double(np.asarray(got, dtype=np.uint16))
        ulp = ulp_bf16(ref16)
    diff = np.abs(g - ref16)
    if fused:
        floor = 2.0 ** -22 * (sab + bias_abs + res_abs + np.abs(ref))
    else:
        floor = 2.0 ** -23 * sab
    bad = ~(diff <= 2.0 * ulp + floor)
    with np.errstate(invalid="ignore", divide="ignore"):
        worst = float(np.nanmax(diff / ulp)) if g.size else 0.0
    res = {"violations": int(bad.sum()), "max_ulps": worst, "count": int(g.size)}
    assert res["violations"] == 0, "%s tolerance violated: %s" % (fmt, res)
    return res
