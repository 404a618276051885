"""Pins of the parameter oracle: generator, Haar rotation, bf16 contract (CPU only)."""
import math

import numpy as np
import pytest

from oracle.params import (SplitMix64, bf16_bits, bf16_value, build_params, gaussian_matrix,
                           haar_from_gaussian)


def test_splitmix64_published_outputs():
    # First outputs of SplitMix64 started from state 0, as produced by the published
    # reference implementation of the generator (Steele, Lea, Flood 2014; Vigna's splitmix64.c).
    g = SplitMix64(0)
    assert [g.next() for _ in range(3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_uniform_and_gaussian_moments():
    g = SplitMix64(12345)
    u = np.array([g.uniform() for _ in range(20000)])
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 4 * math.sqrt(1 / 12 / len(u))
    z = gaussian_matrix(777, 128, 128).ravel()
    n = len(z)
    assert abs(z.mean()) < 4 / math.sqrt(n)
    assert abs(z.var() - 1) < 4 * math.sqrt(2 / n)
    # fourth moment of N(0,1) is 3
    assert abs(np.mean(z ** 4) - 3) < 4 * math.sqrt(96 / n)


def _gram_schmidt_q(G):
    """Modified Gram-Schmidt on the columns: the Q with positive diagonal in G = Q U."""
    d = G.shape[1]
    Q = np.array(G, dtype=np.float64)
    for k in range(d):
        for j in range(k):
            Q[:, k] -= (Q[:, j] @ Q[:, k]) * Q[:, j]
        Q[:, k] /= np.linalg.norm(Q[:, k])
    return Q


@pytest.mark.parametrize("seed", [0, 1, 99])
def test_rotation_is_the_unique_positive_qr_factor(seed):
    p = build_params(seed)
    R = p["R"]
    Q = _gram_schmidt_q(p["G"])
    assert np.abs(R - Q).max() < 1e-9
    U = R.T @ p["G"]
    assert np.abs(np.tril(U, -1)).max() < 1e-9
    assert np.all(np.diag(U) > 0)


@pytest.mark.parametrize("seed", [0, 7])
def test_orthogonality(seed):
    p = build_params(seed)
    I = np.eye(128)
    assert np.abs(p["R"].T @ p["R"] - I).max() < 1e-12
    # the matrix actually applied (bf16 hi + lo) meets the 1e-5 bound
    Re = p["R_eff"]
    assert np.abs(Re.T @ Re - I).max() < 1e-5
    # norm preservation of random vectors through R_eff
    x = np.random.default_rng(seed).standard_normal((64, 128))
    ratio = np.linalg.norm(x @ Re.T, axis=1) / np.linalg.norm(x, axis=1)
    assert np.abs(ratio - 1).max() < 1e-5


def test_single_bf16_rotation_is_not_orthogonal_enough():
    # Why the two-term split exists: one bf16 copy misses the 1e-5 bound by far.
    p = build_params(0)
    Rh = bf16_value(p["r_hi"])
    assert np.abs(Rh.T @ Rh - np.eye(128)).max() > 1e-4


def test_haar_second_moments():
    # For a Haar orthogonal matrix every entry has E[R_ij^2] = 1/d and E[R_ij^4] = 3/(d(d+2)).
    d, n = 32, 4000
    rng = np.random.default_rng(5)
    acc2 = np.zeros((d, d))
    acc4 = np.zeros((d, d))
    for _ in range(n):
        R = haar_from_gaussian(rng.standard_normal((d, d)))
        acc2 += R ** 2
        acc4 += R ** 4
    m2 = acc2 / n
    m4 = acc4 / n
    assert abs(m2.mean() - 1 / d) < 0.01 / d
    assert np.abs(m2 - 1 / d).max() < 0.15 / d
    assert abs(m4.mean() - 3 / (d * (d + 2))) < 0.05 * 3 / (d * (d + 2))
    # without the sign fix Q would not be Haar: its diagonal would be biased negative
    # for LAPACK's convention; with it the mean diagonal is 0.
    diag = np.mean([np.diag(haar_from_gaussian(rng.standard_normal((d, d)))).mean() for _ in range(400)])
    assert abs(diag) < 0.02


def test_bf16_rounding_cases():
    # 1.0; a tie rounds to even; a tie above an odd mantissa rounds up; negative; large.
    vals = [1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 3.0e38, 2 ** -130]
    expect = [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F62, None]
    got = bf16_bits(np.array(vals))
    for g, e in zip(got[:5], expect[:5]):
        assert int(g) == e
    # double rounding through fp32: just above a bf16 tie in fp64, but fp32 rounding lands
    # on the tie, which then goes to even.
    v = 1 + 2 ** -8 + 2 ** -40
    assert int(bf16_bits(np.array([v]))[0]) == 0x3F80
    assert float(bf16_value(np.array([0x3F81], dtype=np.uint16))[0]) == 1 + 2 ** -7


def test_split_reconstructs_to_sixteen_bits():
    p = build_params(0)
    R, Re = p["R"], p["R_eff"]
    rel = np.abs(Re - R) / np.abs(R)
    assert np.quantile(rel, 0.999) < 2 ** -15
    assert np.abs(Re - R).max() < 2 ** -16 * np.abs(R).max()


def test_seeds_give_independent_streams():
    a = build_params(0)
    b = build_params(1)
    assert not np.array_equal(a["r_hi"], b["r_hi"])
    # rotation and sketch come from different streams of the same seed
    assert not np.allclose(a["G"], a["S"])
    # the sketch of seed s is the stream started at 2s + 1, filled row-major
    np.testing.assert_array_equal(b["S"][0, :16], gaussian_matrix(3, 1, 16)[0])
    np.testing.assert_array_equal(b["G"][0, :16], gaussian_matrix(2, 1, 16)[0])
