"""Element-wise comparison of GPU fp16 outputs with the oracle.

Tolerance (stated for this operation): |y - r| <= 2e-3 * |r| + 1e-2 per element,
where r is the oracle's fp16 output and y the GPU's.

Because the exact sums can exceed fp16's range, outputs are split by the
oracle's exact value x (before rounding):
  * finite region, |x| < 65504 * (1 - 2e-3) - 1e-2: y finite and within tol;
  * overflow band, up to 65520 * (1 + 2e-3): y has the sign of x and is either
    +-inf or within 2e-3 * 65504 + 1e-2 of +-65504 (fp32 accumulation may
    land on either side of the rounding threshold 65520);
  * overflow region beyond that: y is sign(x) * inf (fp16 round-to-nearest
    overflows to infinity, it does not saturate).
A NaN in y always fails.
"""
from __future__ import annotations

import numpy as np

RTOL = 2e-3
ATOL = 1e-2
F16_MAX = 65504.0
FINITE_LIMIT = F16_MAX * (1 - RTOL) - ATOL
BAND_LIMIT = 65520.0 * (1 + RTOL)


def check(y16: np.ndarray, r16: np.ndarray, x: np.ndarray, extra_tol=None):
    """Returns (n_violations, max_ratio, detail) where max_ratio is the worst
    |y - r| / tol over the finite region.  ``extra_tol`` (per element) widens
    the tolerance for inputs outside the workload distribution."""
    y = np.asarray(y16, dtype=np.float16).astype(np.float64).ravel()
    r = np.asarray(r16, dtype=np.float16).astype(np.float64).ravel()
    x = np.asarray(x, dtype=np.float64).ravel()
    assert y.shape == r.shape == x.shape
    bad = np.isnan(y)
    ax = np.abs(x)
    fin = ax < FINITE_LIMIT
    band = (ax >= FINITE_LIMIT) & (ax < BAND_LIMIT)
    over = ax >= BAND_LIMIT

    tol = RTOL * np.abs(r) + ATOL
    if extra_tol is not None:
        tol = tol + np.asarray(extra_tol, dtype=np.float64).ravel()
    with np.errstate(invalid="ignore"):
        err = np.where(fin & np.isfinite(y), np.abs(y - r), np.inf)
    ratio = np.where(fin, err / tol, 0.0)
    bad |= fin & (ratio > 1.0)

    sgn_ok = np.sign(y) == np.sign(x)
    near_max = np.abs(np.abs(y) - F16_MAX) <= RTOL * F16_MAX + ATOL
    bad |= band & ~(sgn_ok & (np.isinf(y) | near_max))
    bad |= over & ~(np.isinf(y) & sgn_ok)

    max_ratio = float(ratio[fin].max()) if fin.any() else 0.0
    detail = ""
    if bad.any():
        idx = np.flatnonzero(bad)[:8]
        detail = "; ".join("i=%d y=%r r=%r x=%r" % (i, y[i], r[i], x[i]) for i in idx)
    return int(bad.sum()), max_ratio, detail


def assert_close(y16, r16, x, what="", extra_tol=None):
    n, ratio, detail = check(y16, r16, x, extra_tol)
    assert n == 0, "%s: %d elements out of tolerance (worst finite ratio %.3f): %s" % (
        what, n, ratio, detail)
    return ratio
