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
"""
from __future__ import annotations

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


def lloyd_max_gaussian(bits: int, tol: float = 1e-15, max_iter: int = 100_000):
    """Return (centroids[L], thresholds[L-1], mse, iterations) in fp64 for L = 2**bits levels."""
    if bits < 1 or bits > 8:
        raise ValueError("bits must be in 1..8")
    L = 1 << bits
    c = np.array([-3.0 + 6.0 * (l + 0.5) / L for l in range(L)], dtype=np.float64)
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([-math.inf], t, [math.inf]))
        new_c = np.empty_like(c)
        for l in range(L):
            a, b = edges[l], edges[l + 1]
            new_c[l] = (phi(a) - phi(b)) / cell_mass(a, b)
        delta = float(np.max(np.abs(new_c - c)))
        c = new_c
        if delta < tol:
            break
    t = 0.5 * (c[:-1] + c[1:])
    return c, t, gaussian_mse(c, t), it


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


def codebook_f32(bits: int):
    """The stored tables: fp32 copies of the fp64 levels and thresholds, plus the fp64 MSE."""
    c, t, mse, _ = lloyd_max_gaussian(bits)
    return c.astype(np.float32), t.astype(np.float32), mse
