"""Parity comparator -- TEST INFRASTRUCTURE ONLY (part of the oracle).

Tolerances (readings of the parity rule for this operator; the pages fix FP32
accumulation with final narrowing, page "MatMul Kernel Design", section
"Types and algorithm selection"):

* FLOAT output: ``max |y - o| <= 1e-4 * sqrt(K) * max|A| * max|B|`` where
  ``o`` is the fp64 oracle value and the maxima run over the whole stored A
  and B.
* FLOAT16 / BFLOAT16 output: each element is within 2 units in the last place
  of ``narrow(o)`` (ulp distance measured on the monotone ordering of the
  16-bit patterns), or -- for results so close to zero that the output ulp is
  finer than FP32 accumulation noise -- meets the FLOAT rule above.  The
  number of elements that pass only through the second clause is reported.
* DOUBLE output: ``max |y - o| <= 2 * gamma_K * K * max|A| * max|B|`` with
  ``gamma_K = K u / (1 - K u)``, ``u = 2^-53``.  Products of doubles round,
  so the oracle is no longer exact: the standard bound for a dot product
  formed in floating point with any summation order (Higham, "Accuracy and
  Stability of Numerical Algorithms", 2nd ed., section 3.1) puts both the
  result and the oracle within ``gamma_K * sum_k |a_k b_k|`` of the exact
  value, and ``sum_k |a_k b_k| <= K max|A| max|B|``.
* Gemm (FLOAT, and the second clause for 16-bit outputs): ``|alpha|`` times
  the FLOAT rule, plus ``4 * 2^-24 * (|alpha| K max|A| max|B| + |beta|
  max|C|)`` for the FP32 roundings of ``alpha * sum + beta * c`` (each term
  is at most that large).
* Exact mode (small-integer-valued inputs): ``y == narrow(o)`` bit for bit.
* Special values are judged against ``narrow(o)``, the oracle value rounded
  once to the output type: NaN matches only NaN, and where ``narrow(o)`` is
  an infinity (including a finite sum beyond the type's largest value) only
  that same infinity matches; a finite reference needs a finite result.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import BFLOAT16, DOUBLE, FLOAT, FLOAT16, decode, narrow


def fp32_tolerance(K: int, amax: float, bmax: float) -> float:
    return 1e-4 * math.sqrt(max(int(K), 0)) * float(amax) * float(bmax)


def fp64_tolerance(K: int, amax: float, bmax: float) -> float:
    u = 2.0 ** -53
    k = max(int(K), 0)
    gamma = k * u / (1.0 - k * u)
    return 2.0 * gamma * k * float(amax) * float(bmax)


def gemm_tolerance(K: int, amax: float, bmax: float, cmax: float, alpha: float, beta: float) -> float:
    k = max(int(K), 0)
    return (abs(alpha) * fp32_tolerance(k, amax, bmax)
            + 4.0 * 2.0 ** -24 * (abs(alpha) * k * amax * bmax + abs(beta) * cmax))


def abs_max(x: np.ndarray, dtype: int) -> float:
    """max |x| over stored values (0 for an empty tensor)."""
    if x.size == 0:
        return 0.0
    v = decode(x, dtype) if dtype in (FLOAT16, BFLOAT16) else np.asarray(x, dtype=np.float64)
    return float(np.max(np.abs(v)))


def _key16(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_distance16(y_bits: np.ndarray, r_bits: np.ndarray) -> np.ndarray:
    return np.abs(_key16(y_bits) - _key16(r_bits))


@dataclass
class Report:
    ok: bool
    n: int
    max_abs_err: float
    tolerance: float
    max_ulp: int = 0
    n_fp32_clause: int = 0
    n_bad: int = 0
    detail: str = ""

    def __str__(self) -> str:
        return (f"ok={self.ok} n={self.n} max_abs_err={self.max_abs_err:.3e} tol={self.tolerance:.3e} "
                f"max_ulp={self.max_ulp} fp32_clause={self.n_fp32_clause} bad={self.n_bad} {self.detail}")


def _special_mismatch(yv: np.ndarray, rv: np.ndarray) -> np.ndarray:
    """Elements whose NaN / infinity status differs between the result ``yv``
    and the reference ``rv`` -- the oracle value narrowed to the output type,
    so a finite sum beyond the type's range is expected as that infinity.
    NaN matches only NaN; an infinity matches only the same infinity."""
    nan_bad = np.isnan(yv) != np.isnan(rv)
    inf_y, inf_r = np.isinf(yv), np.isinf(rv)
    inf_bad = (inf_y | inf_r) & ~(inf_y & inf_r & (np.sign(yv) == np.sign(rv)))
    return nan_bad | (inf_bad & ~(np.isnan(yv) | np.isnan(rv)))


def check(y: np.ndarray, o: np.ndarray, dtype: int, K: int, amax: float, bmax: float,
          exact: bool = False, tol: float = None) -> Report:
    """Compare stored results ``y`` (float32 / float64 arrays, or uint16 bit
    patterns) with fp64 oracle values ``o`` of the same shape.  ``tol``
    overrides the absolute rule (Gemm passes ``gemm_tolerance``).

    Every status and distance is taken against ``narrow(o)``, the oracle
    value rounded once to the output type: where that reference is an
    infinity (a finite sum past the type's largest value) the result must be
    the same infinity, and where it is finite the result must be finite and
    within the tolerances; ulps are counted between finite bit patterns."""
    o = np.asarray(o, dtype=np.float64).reshape(-1)
    y = np.asarray(y).reshape(-1)
    if y.size != o.size:
        return Report(False, int(y.size), math.inf, 0.0, detail=f"size {y.size} != {o.size}")
    if tol is None:
        tol = fp64_tolerance(K, amax, bmax) if dtype == DOUBLE else fp32_tolerance(K, amax, bmax)
    if y.size == 0:
        return Report(True, 0, 0.0, tol)
    if dtype in (FLOAT16, BFLOAT16):
        y_bits = y.view(np.uint16) if y.dtype != np.uint16 else y
        yv = decode(y_bits, dtype)
        ref = narrow(o, dtype)
        rv = decode(ref, dtype)
        if exact:
            bad = (y_bits != ref) & ~(np.isnan(yv) & np.isnan(rv))
            finite = np.isfinite(yv) & np.isfinite(rv)
            err = np.where(finite, np.abs(yv - o), 0.0)
            return Report(not bad.any(), int(y.size), float(err.max()), 0.0, n_bad=int(bad.sum()),
                          detail="exact")
        special = _special_mismatch(yv, rv)
        finite = np.isfinite(yv) & np.isfinite(rv)
        err = np.where(finite, np.abs(yv - o), 0.0)
        ulp = np.where(finite, ulp_distance16(y_bits, ref), 0)
        ulp_ok = ulp <= 2
        tol_ok = err <= tol
        bad = special | (finite & ~(ulp_ok | tol_ok))
        return Report(not bad.any(), int(y.size), float(err.max()), tol, max_ulp=int(ulp.max()),
                      n_fp32_clause=int((finite & ~ulp_ok & tol_ok).sum()), n_bad=int(bad.sum()))
    if dtype == FLOAT or dtype == DOUBLE:
        yv = y.astype(np.float64)
        ref = narrow(o, dtype)
        rv = ref.astype(np.float64)
        if exact:
            bad = (y.astype(ref.dtype) != ref) & ~(np.isnan(yv) & np.isnan(rv))
            finite = np.isfinite(yv) & np.isfinite(rv)
            err = np.where(finite, np.abs(yv - o), 0.0)
            return Report(not bad.any(), int(y.size), float(err.max()), 0.0, n_bad=int(bad.sum()),
                          detail="exact")
        special = _special_mismatch(yv, rv)
        finite = np.isfinite(yv) & np.isfinite(rv)
        err = np.where(finite, np.abs(yv - o), 0.0)
        bad = special | (finite & (err > tol))
        return Report(not bad.any(), int(y.size), float(err.max()), tol, n_bad=int(bad.sum()))
    raise ValueError(f"dtype {dtype}")
