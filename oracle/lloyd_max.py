"""Lloyd-Max scalar quantizer for the standard normal law (oracle, fp64).

Page: "Когда в марте 2026 года Google опубликовала статью..." (ai-news.ru), paragraph on
the two ideas of TurboQuant: after the random rotation the coordinates are close to
normal, so the optimal quantizer for that known law (Lloyd-Max) is computed once and
stored, with no calibration.  Page "Google TurboQuant простыми словами", section
"Как работает TurboQuant", step 1: the quantizer is applied to each coordinate on its
own, with no stored quantization parameters.

The codebook targets N(0,1) and is applied to z = sqrt(d) * y, where y is a coordinate
of the rotated unit vector (reading: "близкое к нормальному" means N(0,1) after the
sqrt(d) scaling).

Algorithm (Lloyd's fixed point for a known density): thresholds are midpoints of
neighbouring levels; each level is the conditional mean of its cell.  For N(0,1) the
conditional mean of [a, b) is (phi(a) - phi(b)) / (Phi(b) - Phi(a)).  The density is
log-concave, so the fixed point is unique and any ordered start converges.

Reading for wide codes (the pages ask for 8-bit keys, "K8V4", without saying how the table is
found): Lloyd's iteration contracts ever more slowly as the level count grows (at 6 bits and
up it has not converged after 10^5 steps), so after LLOYD_STEPS steps without convergence the
same fixed-point equations c = F(c) are finished by Newton's method.  F_l depends only on
c_{l-1}, c_l, c_{l+1}, so the Jacobian is tridiagonal:
  dF_l/da = phi(a) (F_l - a) / P_l,   dF_l/db = phi(b) (b - F_l) / P_l,
with a, b the cell's edges (midpoints, so each edge moves by half of either neighbour), and
each Newton step solves (J - I) delta = c - F(c) by tridiagonal elimination.  Codes of 1..4
bits converge within LLOYD_STEPS and never take a Newton step.
"""
from __future__ import annotations

import functools
import math

import numpy as np

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def phi(x: float) -> float:
    """Standard normal density; 0 at +-inf."""
    if math.isinf(x):
        return 0.0
    return _INV_SQRT_2PI * math.exp(-0.5 * x * x)


def cell_mass(a: float, b: float) -> float:
    """P(a <= Z < b) for Z ~ N(0,1), written with erfc so that tail cells keep their digits."""
    if a >= 0.0:
        return 0.5 * (math.erfc(a / _SQRT2) - math.erfc(b / _SQRT2))
    if b <= 0.0:
        return 0.5 * (math.erfc(-b / _SQRT2) - math.erfc(-a / _SQRT2))
    return 1.0 - 0.5 * math.erfc(b / _SQRT2) - 0.5 * math.erfc(-a / _SQRT2)


LLOYD_STEPS = 1000       # Lloyd steps before Newton takes over
NEWTON_TOL = 1e-11       # Newton stops once its step is below this (fp64 noise is near 1e-13)
NEWTON_STEPS = 50


def lloyd_map(c: np.ndarray):
    """One Lloyd step: the conditional means F(c) of the cells whose edges are the midpoints of
    c, and the derivatives of each F_l with respect to its lower and upper edge."""
    L = len(c)
    t = 0.5 * (c[:-1] + c[1:])
    edges = np.concatenate(([-math.inf], t, [math.inf]))
    f = np.empty(L)
    d_lo = np.zeros(L)
    d_hi = np.zeros(L)
    for l in range(L):
        a, b = edges[l], edges[l + 1]
        m = cell_mass(a, b)
        f[l] = (phi(a) - phi(b)) / m
        if not math.isinf(a):
            d_lo[l] = phi(a) * (f[l] - a) / m
        if not math.isinf(b):
            d_hi[l] = phi(b) * (b - f[l]) / m
    return f, d_lo, d_hi


def solve_tridiagonal(sub, diag, sup, rhs):
    """x with sub[i] x[i-1] + diag[i] x[i] + sup[i] x[i+1] = rhs[i] (Thomas elimination)."""
    n = len(diag)
    cp = np.zeros(n)
    dp = np.zeros(n)
    cp[0] = sup[0] / diag[0] if n > 1 else 0.0
    dp[0] = rhs[0] / diag[0]
    for i in range(1, n):
        m = diag[i] - sub[i] * cp[i - 1]
        cp[i] = sup[i] / m if i < n - 1 else 0.0
        dp[i] = (rhs[i] - sub[i] * dp[i - 1]) / m
    x = np.zeros(n)
    x[-1] = dp[-1]
    for i in range(n - 2, -1, -1):
        x[i] = dp[i] - cp[i] * x[i + 1]
    return x


def lloyd_max_gaussian(bits: int, tol: float = 1e-15):
    """Return (centroids[L], thresholds[L-1], mse, steps) in fp64 for L = 2**bits levels; steps
    counts Lloyd steps plus Newton steps."""
    if bits < 1 or bits > 8:
        raise ValueError("bits must be in 1..8")
    L = 1 << bits
    c = np.array([-3.0 + 6.0 * (l + 0.5) / L for l in range(L)], dtype=np.float64)
    steps = 0
    converged = False
    while steps < LLOYD_STEPS:
        steps += 1
        f, _, _ = lloyd_map(c)
        delta = float(np.max(np.abs(f - c)))
        c = f
        if delta < tol:
            converged = True
            break
    if not converged:
        for _ in range(NEWTON_STEPS):
            steps += 1
            f, d_lo, d_hi = lloyd_map(c)
            # J has 0.5 d_lo below the diagonal, 0.5 (d_lo + d_hi) on it, 0.5 d_hi above it
            delta = solve_tridiagonal(0.5 * d_lo, 0.5 * (d_lo + d_hi) - 1.0, 0.5 * d_hi, c - f)
            c = c + delta
            if float(np.max(np.abs(delta))) < NEWTON_TOL:
                break
        # N(0,1) is symmetric, so is its quantizer: the fp64 noise of the solve (~1e-13) is
        # averaged out of the mirror pairs, which puts the middle threshold exactly at 0 (a
        # zero coordinate then takes code 2^(b-1), as with the narrow tables)
        c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    return c, t, gaussian_mse(c, t), steps


def gaussian_mse(c: np.ndarray, t: np.ndarray) -> float:
    """E[(Z - q(Z))^2] for Z ~ N(0,1) when every level is its cell's conditional mean.

    With centroid levels, E[(Z - q)^2] = E[Z^2] - sum_l P_l c_l^2 and P_l c_l =
    phi(a_l) - phi(b_l), hence 1 - sum_l (phi(a_l) - phi(b_l))^2 / P_l.
    """
    edges = np.concatenate(([-math.inf], np.asarray(t, dtype=np.float64), [math.inf]))
    s = 0.0
    for l in range(len(c)):
        a, b = edges[l], edges[l + 1]
        m = cell_mass(a, b)
        s += (phi(a) - phi(b)) ** 2 / m
    return 1.0 - s


@functools.lru_cache(maxsize=None)
def _codebook_f32(bits: int):
    c, t, mse, _ = lloyd_max_gaussian(bits)
    return c.astype(np.float32), t.astype(np.float32), mse


def codebook_f32(bits: int):
    """The stored tables: fp32 copies of the fp64 levels and thresholds, plus the fp64 MSE
    (computed once per width; each call returns fresh arrays)."""
    c, t, mse = _codebook_f32(bits)
    return c.copy(), t.copy(), mse
