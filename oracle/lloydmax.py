"""Oracle: Lloyd-Max quantizer for the standard normal distribution.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[PolarQuant] section 2 scales the rotated coordinates to N(0, 1) and quantizes
them with the MSE-optimal (Lloyd-Max) centroids for that distribution; the
table is stored in float32.  Lloyd-Max optimality means the two conditions

    tau_k = (c_k + c_{k+1}) / 2                  (nearest-neighbour cells)
    c_k   = E[X | tau_{k-1} < X < tau_k]         (centroid of each cell)

with tau_{-1} = -inf, tau_{L-1} = +inf.  For N(0,1) the conditional mean of
(a, b) is (phi(a) - phi(b)) / (Phi(b) - Phi(a)).  The solution is symmetric,
so only the positive half is solved; for even L the middle threshold is 0.
The fixed-point iteration of the two conditions is run first and a Newton
root solve of the same conditions finishes it (plain iteration converges very
slowly for 32 levels).
"""

from __future__ import annotations

import numpy as np
from scipy import optimize, special

_SQRT2 = np.sqrt(2.0)
_INV_SQRT2PI = 1.0 / np.sqrt(2.0 * np.pi)


def _phi(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        out = _INV_SQRT2PI * np.exp(-0.5 * x * x)
    return np.where(np.isinf(x), 0.0, out)


def _upper_tail(x):
    """1 - Phi(x), accurate in the upper tail."""
    return 0.5 * special.erfc(np.asarray(x, dtype=np.float64) / _SQRT2)


def _cell_mean(a, b):
    """E[X | a < X < b] for X ~ N(0,1), 0 <= a < b <= inf."""
    p = _upper_tail(a) - _upper_tail(b)
    return (_phi(a) - _phi(b)) / p


def _positive_half(levels: int):
    if levels < 2 or levels % 2:
        raise ValueError("an even number of levels >= 2 is required")
    return levels // 2


def _thresholds_from(cpos):
    """Positive thresholds [0, mid_1, ..., inf] for positive centroids cpos."""
    mids = 0.5 * (cpos[:-1] + cpos[1:])
    return np.concatenate([[0.0], mids, [np.inf]])


def _residual(cpos):
    t = _thresholds_from(cpos)
    return cpos - _cell_mean(t[:-1], t[1:])


def lloyd_max_gaussian(bits: int, tol: float = 1e-13, max_iter: int = 20000):
    """Centroids (ascending, L = 2^bits), thresholds (L-1, ascending) and MSE."""
    levels = 1 << bits
    half = _positive_half(levels)
    # start: centroids of equal-probability cells of the positive half
    q = (np.arange(half) + 0.5) / half
    cpos = np.sqrt(2.0) * special.erfinv(q)  # quantiles of |X| (half-normal)
    for _ in range(max_iter):
        t = _thresholds_from(cpos)
        new = _cell_mean(t[:-1], t[1:])
        if np.max(np.abs(new - cpos)) <= tol:
            cpos = new
            break
        cpos = new
    if np.max(np.abs(_residual(cpos))) > tol:
        sol = optimize.root(_residual, cpos, method="hybr", tol=1e-15)
        cpos = sol.x
    cpos = np.sort(cpos)
    cent = np.concatenate([-cpos[::-1], cpos])
    tpos = _thresholds_from(cpos)[:-1]  # 0 and the positive midpoints
    thr = np.concatenate([-tpos[:0:-1], tpos])
    return cent, thr, gaussian_mse(cent, thr)


def gaussian_mse(centroids, thresholds) -> float:
    """E[(X - Q(X))^2] for X ~ N(0,1), cell k = (tau_{k-1}, tau_k) -> c_k.

    Uses E[X^2; a<X<b] = P + a phi(a) - b phi(b) and E[X; a<X<b] = phi(a) - phi(b)."""
    c = np.asarray(centroids, dtype=np.float64)
    t = np.concatenate([[-np.inf], np.asarray(thresholds, dtype=np.float64), [np.inf]])
    a, b = t[:-1], t[1:]
    p = special.ndtr(b) - special.ndtr(a)
    ex = _phi(a) - _phi(b)
    with np.errstate(invalid="ignore"):
        ax = np.where(np.isinf(a), 0.0, a * _phi(a))
        bx = np.where(np.isinf(b), 0.0, b * _phi(b))
    ex2 = p + ax - bx
    return float(np.sum(ex2 - 2.0 * c * ex + c * c * p))


def stationarity_residual(centroids) -> float:
    """max |c_k - E[X | cell k]| for the nearest-neighbour cells of centroids."""
    c = np.asarray(centroids, dtype=np.float64)
    t = np.concatenate([[-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]])
    p = special.ndtr(t[1:]) - special.ndtr(t[:-1])
    means = (_phi(t[:-1]) - _phi(t[1:])) / p
    return float(np.max(np.abs(c - means)))
