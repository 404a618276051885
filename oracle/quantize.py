"""Quantize-on-write of key / value vectors (oracle, fp64).

Pages: "Когда в марте 2026 года Google опубликовала статью..." (ai-news.ru): rotate by a
random orthogonal matrix, then apply the precomputed Lloyd-Max quantizer to each
coordinate, then the QJL correction of the residual; no per-group scale metadata.
"Google TurboQuant простыми словами", section "Как работает TurboQuant", step 2: QJL
projects the residual with a Johnson-Lindenstrauss transform and keeps one sign bit
per row, which makes the inner-product estimate unbiased.  Section "Бенчмарки
TurboQuant", list "Из независимых реализаций": 52 bytes per 128 values (48 bytes of
3-bit codes plus a 4-byte side value), read here as one fp32 norm per vector.

Steps per vector x (d coordinates, taken exactly as given):
  n = ||x||_2;  y = R_eff x / n;  z = sqrt(d) y
  idx_j = #{l : z_j >= t_l}            (ties go to the upper cell)
  keys with the sign sketch and b >= 1:  r = y - c[idx] / sqrt(d);  gamma = ||r||_2
  keys with the sign sketch and b == 0:  r = y;  gamma = 1 (not stored)
  u = S_b r;  sigma_j = 1 iff u_j >= 0
A zero vector (n = 0) gets idx = L/2 everywhere (z = 0 sits on the middle threshold),
gamma = 0 and sigma = 1: its stored norm makes its key score and value contribution 0.
"""
from __future__ import annotations

import math

import numpy as np


def kappa(m: int) -> float:
    """Scale of the sign estimate: E[(g.a) sign(g.b)] = sqrt(2/pi) <a,b>/||b|| for g ~ N(0,I),
    so sqrt(pi/2)/m * ||r|| * <S q, sign(S r)> has mean <q, r> over the m Gaussian rows."""
    return math.sqrt(math.pi / 2.0) / m


def quantize(x, R_eff, centroids=None, thresholds=None, S_b=None, force_idx=None, force_mask=None):
    """Quantize rows of x.

    x          [N, d] values (any float dtype; used exactly, in fp64)
    R_eff      [d, d] rotation actually applied (fp64)
    centroids  fp32 levels (length L) or None when the vectors get no scalar code (b = 0)
    thresholds fp32 decision thresholds (length L-1)
    S_b        [m, d] sketch matrix (fp64 values of the bf16 entries) or None (no sign sketch)
    force_idx / force_mask: optional [N, d] codes and mask; where the mask is set the given
              code replaces the computed one before the residual is formed (used to follow
              the other side's choice for coordinates that sit on a threshold).
    Returns a dict of idx (uint8 [N,d]), sign (bool [N,m]), n, gamma (fp64 [N]), z, u, r.
    """
    x = np.asarray(x, dtype=np.float64)
    N, d = x.shape
    n = np.sqrt(np.sum(x * x, axis=1))
    zero = n == 0.0
    safe_n = np.where(zero, 1.0, n)
    y = (x @ R_eff.T) / safe_n[:, None]
    y[zero] = 0.0
    z = math.sqrt(d) * y
    out = {"n": n, "z": z}
    if centroids is not None:
        c = np.asarray(centroids, dtype=np.float32).astype(np.float64)
        t = np.asarray(thresholds, dtype=np.float32).astype(np.float64)
        idx = np.searchsorted(t, z, side="right")
        if force_idx is not None:
            idx = np.where(force_mask, force_idx, idx)
        out["idx"] = idx.astype(np.uint8)
        r = y - c[idx] / math.sqrt(d)
    else:
        r = y
    if S_b is not None:
        if centroids is not None:
            gamma = np.sqrt(np.sum(r * r, axis=1))
            gamma[zero] = 0.0
        else:
            gamma = np.ones(N)
        u = r @ np.asarray(S_b, dtype=np.float64).T
        u[zero] = 0.0
        out["gamma"] = gamma
        out["u"] = u
        out["sign"] = u >= 0.0
        out["r"] = r
    return out


def threshold_band(z, thresholds, rel=1e-5):
    """True where z lies within rel * max(1, |t_l|) of some threshold t_l (fp32 thresholds).

    Only the thresholds next to z (below and above it) are tested: thresholds are sorted and
    spaced far wider than two band widths (the narrowest gap, at 8 bits, is ~0.016 against
    bands of at most ~1e-4 for rel = 1e-5), so no farther threshold can reach z."""
    t = np.asarray(thresholds, dtype=np.float32).astype(np.float64)
    z = np.asarray(z, dtype=np.float64)
    assert rel * max(1.0, float(np.abs(t).max())) * 2 < float(np.min(np.diff(t))) if len(t) > 1 else True
    i = np.searchsorted(t, z)
    lo = t[np.clip(i - 1, 0, len(t) - 1)]
    hi = t[np.clip(i, 0, len(t) - 1)]
    return ((np.abs(z - lo) <= rel * np.maximum(1.0, np.abs(lo))) |
            (np.abs(z - hi) <= rel * np.maximum(1.0, np.abs(hi))))


def sign_band(u, r_norm, rel=1e-5):
    """True where the sketch value u_j lies within rel * ||r|| of the decision point 0."""
    return np.abs(u) <= rel * np.asarray(r_norm)[:, None]


def dequantize(q, R_eff, centroids=None, S_b=None):
    """Vector the codes stand for: n R_eff^T (c[idx]/sqrt(d) + gamma kappa S_b^T (2 sigma - 1))."""
    n = q["n"]
    d = R_eff.shape[0]
    w = np.zeros((len(n), d))
    if centroids is not None:
        c = np.asarray(centroids, dtype=np.float32).astype(np.float64)
        w += c[q["idx"].astype(np.int64)] / math.sqrt(d)
    if S_b is not None:
        m = S_b.shape[0]
        pm = np.where(q["sign"], 1.0, -1.0)
        w += (q["gamma"] * kappa(m))[:, None] * (pm @ S_b)
    return n[:, None] * (w @ R_eff)
