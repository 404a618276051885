"""Pins of the quantize-on-write oracle (CPU only)."""
import math
import os

import numpy as np
import pytest

from oracle.attention import key_scores
from oracle.lloyd_max import codebook_f32, lloyd_max_gaussian
from oracle.params import build_params
from oracle.quantize import dequantize, kappa, quantize, sign_band, threshold_band

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
P0 = build_params(0)


def _figures():
    out = {}
    for line in open(os.path.join(GOLDEN, "pages_figures.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()[:2]
            out[k] = float(v)
    return out


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
def test_threshold_count_is_nearest_centroid(bits):
    c, t, _ = codebook_f32(bits)
    rng = np.random.default_rng(bits)
    z = rng.standard_normal(200000) * 1.5
    idx = np.searchsorted(t.astype(np.float64), z, side="right")
    brute = np.argmin(np.abs(z[:, None] - c.astype(np.float64)[None, :]), axis=1)
    far = ~threshold_band(z[None, :], t, rel=1e-6)[0]
    np.testing.assert_array_equal(idx[far], brute[far])
    # a value exactly on a threshold goes to the upper cell
    on = np.searchsorted(t.astype(np.float64), t.astype(np.float64), side="right")
    np.testing.assert_array_equal(on, np.arange(1, len(t) + 1))


def test_quantize_uses_codes_of_the_rotated_scaled_vector():
    c, t, _ = codebook_f32(3)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 128))
    q = quantize(x, P0["R_eff"], c, t, None)
    y = (x @ P0["R_eff"].T) / np.linalg.norm(x, axis=1)[:, None]
    z = math.sqrt(128) * y
    brute = np.argmin(np.abs(z[..., None] - c.astype(np.float64)), axis=-1)
    np.testing.assert_array_equal(q["idx"], brute)
    np.testing.assert_allclose(q["n"], np.linalg.norm(x, axis=1), rtol=1e-15)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_mirror_symmetry(bits):
    c, t, _ = codebook_f32(bits)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((200, 128))
    a = quantize(x, P0["R_eff"], c, t, None)
    b = quantize(-x, P0["R_eff"], c, t, None)
    off = ~threshold_band(a["z"], t)
    L = 1 << bits
    np.testing.assert_array_equal(b["idx"][off], (L - 1 - a["idx"].astype(int))[off])


def test_zero_vector():
    kc, kt, _ = codebook_f32(2)
    x = np.zeros((2, 128))
    x[1, 5] = 1.0
    q = quantize(x, P0["R_eff"], kc, kt, P0["S_b"])
    assert q["n"][0] == 0.0 and np.all(q["idx"][0] == 2)
    assert q["gamma"][0] == 0.0 and np.all(q["sign"][0])
    assert q["n"][1] == 1.0 and q["gamma"][1] > 0


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 6, 8])
def test_empirical_mse_on_unit_vectors(bits):
    # Normalized squared error ||x - xhat||^2 / ||x||^2 of random unit vectors (d = 128)
    # through the whole value path: within [-3 %, +0.5 %] of the Gaussian optimum D_b
    # (coordinates of a rotated unit vector have lighter tails than N(0,1)).
    c, t, _ = codebook_f32(bits)
    _, _, D, _ = lloyd_max_gaussian(bits)
    rng = np.random.default_rng(100 + bits)
    x = rng.standard_normal((40000, 128))
    x /= np.linalg.norm(x, axis=1)[:, None]
    q = quantize(x, P0["R_eff"], c, t, None)
    xh = dequantize(q, P0["R_eff"], c, None)
    mse = np.mean(np.sum((x - xh) ** 2, axis=1))
    assert -0.03 <= mse / D - 1 <= 0.005
    figs = _figures()
    if bits == 3:
        assert abs(mse - figs["mse_3bit"]) < 0.0005
    if bits == 4:
        assert abs(mse - figs["mse_4bit"]) < 0.0005


def _sketch_draws(n_draws, m, d, seed):
    rng = np.random.default_rng(seed)
    for _ in range(n_draws):
        yield rng.standard_normal((m, d))


@pytest.mark.parametrize("k_bits", [0, 2])
def test_qjl_estimate_is_unbiased_over_sketches(k_bits):
    # Over many independent Gaussian sketches the mean key score equals the exact inner
    # product <R_eff q, R_eff x> (zero bias of the sign correction).  With k_bits = 0
    # this is the plain 1-bit Johnson-Lindenstrauss inner-product estimator.
    d = m = 128
    rng = np.random.default_rng(42)
    x = rng.standard_normal((1, d)) * 3.0
    qv = rng.standard_normal((1, d))
    kc, kt = (None, None) if k_bits == 0 else codebook_f32(k_bits)[:2]
    Re = P0["R_eff"]
    target = float(((qv @ Re.T) @ (x @ Re.T).T)[0, 0])
    n_draws = 20000
    est = np.empty(n_draws)
    for i, S in enumerate(_sketch_draws(n_draws, m, d, 7 + k_bits)):
        k = quantize(x, Re, kc, kt, S)
        est[i] = key_scores(qv, Re, k, kc, S)[0, 0]
    se = est.std(ddof=1) / math.sqrt(n_draws)
    assert abs(est.mean() - target) < 4 * se
    # variance closed form: n^2 gamma^2 / m (pi/2 ||q1||^2 - <q1, r/||r||>^2)
    k = quantize(x, Re, kc, kt, np.eye(m, d))
    q1 = (qv @ Re.T)[0]
    r = k["r"][0]
    gamma = np.linalg.norm(r) if k_bits else 1.0
    alpha = q1 @ r / np.linalg.norm(r)
    var = k["n"][0] ** 2 * gamma ** 2 / m * (math.pi / 2 * (q1 @ q1) - alpha ** 2)
    assert abs(est.var(ddof=1) / var - 1) < 0.05


def test_kappa():
    assert kappa(128) == math.sqrt(math.pi / 2) / 128


def test_sign_band_and_threshold_band_shapes():
    c, t, _ = codebook_f32(2)
    z = np.array([[t[0], t[0] + 2e-5, 0.0, 5.0]])
    b = threshold_band(z, t)
    assert b.tolist() == [[True, False, True, False]]
    u = np.array([[0.0, 1e-6, -1e-6, 1.0]])
    assert sign_band(u, np.array([1.0])).tolist() == [[True, True, True, False]]
