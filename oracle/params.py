"""Seeded parameters of the method: random orthogonal rotation and the QJL sketch (oracle).

Pages: "Когда в марте 2026 года Google опубликовала статью..." (ai-news.ru), paragraph on
the first idea (multiply the vector by a random orthogonal matrix before quantizing);
"Google TurboQuant простыми словами", section "Как работает TurboQuant", step 2 (QJL uses
a Johnson-Lindenstrauss random projection and one extra bit).  The pages say only
"random"; a fully specified generator is this repo's reading so that two independent
implementations produce the same matrices:

* Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; the 64-bit finalizer constants as published there).  The
  rotation stream starts from state 2*seed, the sketch stream from 2*seed + 1.
* Uniform: u = (next() >> 11) * 2**-53.  Gaussians: Box-Muller on pairs (u1, u2) with
  u1 replaced by 1 - u1, giving r*cos(2*pi*u2) then r*sin(2*pi*u2), r = sqrt(-2 ln u1);
  matrices are filled row-major.
* Rotation: G (d x d, rotation stream) = Q U (QR); R = Q diag(sign U_ii), sign 0 -> +1.
  This is a Haar-distributed orthogonal matrix, applied as y = R x.
* Hadamard rotation mode (page "Google TurboQuant простыми словами", section on TurboQuant
  in llama.cpp: the rotation sped up through the Hadamard transform; read as the randomized
  Hadamard transform): R = H diag(s) / sqrt(d), H the Sylvester Hadamard matrix
  (H_ij = (-1)^popcount(i & j)), s_j = -1 when the top bit of the j-th output of the
  rotation stream is set, else +1.  y = R x flips signs, then applies the Walsh-Hadamard
  transform; R is exactly orthogonal.
* Precision contract (Haar mode): R_hi = bf16(R), R_lo = bf16(R - R_hi) (difference in
  fp64); R_eff = R_hi + R_lo is the matrix both sides apply.  bf16(v) rounds v to fp32 (ties
  to even) and then to bf16 (ties to even).
* Precision contract (Hadamard mode): H diag(s) has entries +-1, exact in bf16, so the
  rotation needs no split: R_hi holds H diag(s), R_lo is zero, and R_eff = R exactly (the
  factor 1/sqrt(d) is a scale, applied by each side in its own arithmetic).
* Sketch: S (m x d, m = d) i.i.d. N(0,1) from the sketch stream; S_b = bf16(S) is the
  matrix both sides apply.
"""
from __future__ import annotations

import math

import numpy as np

MASK64 = (1 << 64) - 1


class SplitMix64:
    """SplitMix64 generator over Python integers (exact 64-bit arithmetic)."""

    GAMMA = 0x9E3779B97F4A7C15

    def __init__(self, state: int):
        self.state = state & MASK64

    def next(self) -> int:
        self.state = (self.state + self.GAMMA) & MASK64
        z = self.state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        return z ^ (z >> 31)

    def uniform(self) -> float:
        return (self.next() >> 11) * (2.0 ** -53)


def gaussian_matrix(state: int, rows: int, cols: int) -> np.ndarray:
    """rows x cols i.i.d. N(0,1) by Box-Muller, filled row-major, from a SplitMix64 stream."""
    g = SplitMix64(state)
    n = rows * cols
    out = []
    while len(out) < n:
        u1 = 1.0 - g.uniform()
        u2 = g.uniform()
        r = math.sqrt(-2.0 * math.log(u1))
        out.append(r * math.cos(2.0 * math.pi * u2))
        out.append(r * math.sin(2.0 * math.pi * u2))
    return np.array(out[:n], dtype=np.float64).reshape(rows, cols)


def haar_from_gaussian(G: np.ndarray) -> np.ndarray:
    """Q diag(sign U_ii) from the QR factorization G = Q U (library QR as the step)."""
    Q, U = np.linalg.qr(G)
    s = np.sign(np.diag(U))
    s[s == 0] = 1.0
    return Q * s[None, :]


def to_f32(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def bf16_bits(v) -> np.ndarray:
    """bf16 bit patterns (uint16) of v: round to fp32 (ties to even), then to bf16 (ties to even)."""
    f = np.ascontiguousarray(to_f32(v))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    nan = np.isnan(f)
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """fp64 value of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def hadamard_signs(state: int, d: int) -> np.ndarray:
    """s_j = -1 if the top bit of the j-th SplitMix64 output is set, else +1."""
    g = SplitMix64(state)
    return np.array([-1.0 if (g.next() >> 63) else 1.0 for _ in range(d)])


def sylvester_hadamard(d: int) -> np.ndarray:
    """H_ij = (-1)^popcount(i & j) for i, j < d (d a power of two)."""
    i = np.arange(d)
    parity = np.array([[bin(a & b).count("1") & 1 for b in i] for a in i])
    return np.where(parity == 1, -1.0, 1.0)


ROTATIONS = ("haar", "hadamard")


def build_params(seed: int, d: int = 128, m: int = None, rotation: str = "haar"):
    """Return dict with R (fp64), R_hi/R_lo/S_b bit patterns and their fp64 values, R_eff."""
    m = d if m is None else m
    if rotation == "haar":
        G = gaussian_matrix((2 * seed) & MASK64, d, d)
        R = haar_from_gaussian(G)
    elif rotation == "hadamard":
        G = None
        Hs = sylvester_hadamard(d) * hadamard_signs((2 * seed) & MASK64, d)[None, :]
        R = Hs / math.sqrt(d)
    else:
        raise ValueError(f"rotation must be one of {ROTATIONS}")
    if rotation == "hadamard":
        r_hi = bf16_bits(Hs)
        r_lo = np.zeros((d, d), dtype=np.uint16)
        R_eff = R
    else:
        r_hi = bf16_bits(R)
        r_lo = bf16_bits(R - bf16_value(r_hi))
        R_eff = bf16_value(r_hi) + bf16_value(r_lo)
    S = gaussian_matrix((2 * seed + 1) & MASK64, m, d)
    s_b = bf16_bits(S)
    return {
        "G": G, "R": R, "S": S,
        "r_hi": r_hi, "r_lo": r_lo, "s_b": s_b,
        "R_eff": R_eff, "S_b": bf16_value(s_b),
    }
