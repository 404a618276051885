"""Pins of the Lloyd-Max oracle against closed forms, quadrature, textbook tables and the
figures printed on the pages (CPU only)."""
import math
import os

import numpy as np
import pytest
from scipy import integrate

from oracle.lloyd_max import codebook_f32, lloyd_max_gaussian

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pages_figures():
    out = {}
    with open(os.path.join(GOLDEN, "pages_figures.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = line.split()[:2]
                out[k] = float(v)
    return out


def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


def test_one_bit_levels_closed_form():
    # For one bit the cells are the half-lines; the conditional mean of |Z| is sqrt(2/pi).
    c, t, mse, _ = lloyd_max_gaussian(1)
    assert abs(c[1] - math.sqrt(2 / math.pi)) < 1e-12
    assert abs(c[0] + math.sqrt(2 / math.pi)) < 1e-12
    assert t[0] == 0.0
    assert abs(mse - (1 - 2 / math.pi)) < 1e-12


@pytest.mark.parametrize("bits,printed", [(1, 0.3634), (2, 0.1175), (3, 0.03454), (4, 0.009497)])
def test_mse_matches_printed_optimum(bits, printed):
    # Distortions of the optimal Gaussian quantizers at 1..4 bits as stated for this path.
    _, _, mse, _ = lloyd_max_gaussian(bits)
    assert abs(mse - printed) / printed < 1e-3


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_centroid_condition_by_quadrature(bits):
    # Each level is the conditional mean of its cell, integrated numerically (independent of
    # the erfc closed form used by the oracle), and the MSE integral agrees.
    c, t, mse, _ = lloyd_max_gaussian(bits)
    edges = [-math.inf] + list(t) + [math.inf]
    total = 0.0
    for l in range(len(c)):
        a, b = edges[l], edges[l + 1]
        m0 = integrate.quad(_phi, a, b, epsabs=1e-14, epsrel=1e-13)[0]
        m1 = integrate.quad(lambda x: x * _phi(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(m1 / m0 - c[l]) < 1e-9
        total += integrate.quad(lambda x: (x - c[l]) ** 2 * _phi(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
    assert abs(total - mse) < 1e-9


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_thresholds_are_midpoints_and_symmetric(bits):
    c, t, _, _ = lloyd_max_gaussian(bits)
    L = len(c)
    assert np.all(np.diff(c) > 0)
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=0)
    np.testing.assert_allclose(c, -c[::-1], atol=1e-13)
    assert t[L // 2 - 1] == 0.0


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_local_optimality(bits):
    # Moving any level or threshold a little raises the distortion (quadrature).
    c, t, mse, _ = lloyd_max_gaussian(bits)

    def distortion(cc, tt):
        edges = [-math.inf] + list(tt) + [math.inf]
        return sum(integrate.quad(lambda x: (x - cc[l]) ** 2 * _phi(x), edges[l], edges[l + 1])[0]
                   for l in range(len(cc)))

    for l in range(len(c)):
        cc = c.copy()
        cc[l] += 1e-3
        assert distortion(cc, t) > mse
    for l in range(len(t)):
        tt = t.copy()
        tt[l] += 1e-3
        assert distortion(c, tt) > mse


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_distortion_rate_bounds(bits):
    # The pages: within about 2.7x of the theoretical minimum.  Read as the Gaussian
    # distortion-rate bound 4**-b below and sqrt(3)*pi/2 * 4**-b (the high-rate
    # optimal-quantizer constant, ~2.72) above.
    figs = _pages_figures()
    _, _, mse, _ = lloyd_max_gaussian(bits)
    lower = 4.0 ** -bits
    assert lower <= mse <= math.sqrt(3) * math.pi / 2 * lower
    assert mse / lower < figs["near_optimal_factor"] + 0.05


def test_classical_tables():
    # Max (1960), "Quantizing for minimum distortion", IRE Trans. Inform. Theory IT-6,
    # optimal Gaussian quantizer levels to three decimals.
    c2, t2, _, _ = lloyd_max_gaussian(2)
    np.testing.assert_allclose(c2[2:], [0.4528, 1.510], atol=1e-3)
    np.testing.assert_allclose(t2[2:], [0.9816], atol=1e-3)
    c3, t3, _, _ = lloyd_max_gaussian(3)
    np.testing.assert_allclose(c3[4:], [0.2451, 0.7560, 1.344, 2.152], atol=1e-3)
    np.testing.assert_allclose(t3[4:], [0.5006, 1.050, 1.748], atol=1e-3)


def test_tables_stored_as_fp32():
    c, t, mse = codebook_f32(3)
    c64, t64, mse64, _ = lloyd_max_gaussian(3)
    assert c.dtype == np.float32 and t.dtype == np.float32
    np.testing.assert_array_equal(c, c64.astype(np.float32))
    np.testing.assert_array_equal(t, t64.astype(np.float32))
    assert mse == mse64
