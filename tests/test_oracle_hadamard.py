"""Pins of the oracle's Hadamard rotation mode (R = H diag(s) / sqrt(d)), independent of its
own construction: a fast Walsh-Hadamard transform written here as butterflies, the Kronecker
construction of H, exact orthogonality, the sign stream, and the distortion of the whole
value path.  (Page "Google TurboQuant простыми словами", section on TurboQuant in llama.cpp:
the rotation sped up through the Hadamard transform.)"""
import math

import numpy as np
import pytest

from oracle.lloyd_max import codebook_f32, lloyd_max_gaussian
from oracle.params import SplitMix64, bf16_value, build_params
from oracle.pipeline import Oracle
from oracle.quantize import dequantize, quantize

D = 128


def fwht(x):
    """Unnormalized Walsh-Hadamard transform along the last axis, in place butterflies."""
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        for i in range(0, n, 2 * h):
            a = y[..., i:i + h].copy()
            b = y[..., i + h:i + 2 * h].copy()
            y[..., i:i + h] = a + b
            y[..., i + h:i + 2 * h] = a - b
        h *= 2
    return y


def kronecker_hadamard(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


@pytest.mark.parametrize("seed", [0, 1, 777])
def test_rotation_is_sign_flip_then_walsh_hadamard(seed):
    p = build_params(seed, rotation="hadamard")
    g = SplitMix64(2 * seed)
    s = np.array([-1.0 if (g.next() >> 63) else 1.0 for _ in range(D)])
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((5, D))
    np.testing.assert_allclose(x @ p["R"].T, fwht(x * s) / math.sqrt(D), rtol=0, atol=1e-13)
    # H itself: the Kronecker construction, and R = H diag(s) / sqrt(d) entry by entry
    H = kronecker_hadamard(D)
    np.testing.assert_array_equal(p["R"] * math.sqrt(D), H * s[None, :])
    # both signs occur (the stream is not degenerate) and the first row is s / sqrt(d)
    assert 0 < np.sum(s > 0) < D
    np.testing.assert_array_equal(p["R"][0] * math.sqrt(D), s)


@pytest.mark.parametrize("seed", [0, 9])
def test_applied_rotation_is_exact_and_needs_no_split(seed):
    # H diag(s) has entries +-1, exact in bf16: the stored hi term is H diag(s) itself (bf16
    # patterns 0x3F80 / 0xBF80), the lo term is zero, and the applied rotation is R exactly
    p = build_params(seed, rotation="hadamard")
    g = SplitMix64(2 * seed)
    s = np.array([-1.0 if (g.next() >> 63) else 1.0 for _ in range(D)])
    Hs = kronecker_hadamard(D) * s[None, :]
    np.testing.assert_array_equal(p["r_hi"], np.where(Hs > 0, 0x3F80, 0xBF80).astype(np.uint16))
    np.testing.assert_array_equal(p["r_lo"], np.zeros((D, D), dtype=np.uint16))
    np.testing.assert_array_equal(bf16_value(p["r_hi"]), Hs)
    np.testing.assert_array_equal(p["R_eff"], p["R"])
    # orthogonal to fp64 rounding: (H diag(s))^T (H diag(s)) = d I exactly, and R = that / sqrt(d)
    np.testing.assert_array_equal(Hs.T @ Hs, D * np.eye(D))
    assert np.abs(p["R_eff"].T @ p["R_eff"] - np.eye(D)).max() < 1e-15


def test_sketch_and_codebooks_do_not_depend_on_the_rotation():
    a, b = build_params(5), build_params(5, rotation="hadamard")
    np.testing.assert_array_equal(a["s_b"], b["s_b"])
    assert not np.array_equal(a["r_hi"], b["r_hi"])
    with pytest.raises(ValueError):
        build_params(0, rotation="dct")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_distortion_of_random_unit_vectors(bits):
    # Random unit vectors through the value path with the Hadamard rotation: the rotated
    # coordinates are close to N(0, 1/d), so the normalized MSE is close to the Gaussian
    # optimum D_b, as with the Haar rotation.
    c, t, _ = codebook_f32(bits)
    _, _, Db, _ = lloyd_max_gaussian(bits)
    p = build_params(3, rotation="hadamard")
    rng = np.random.default_rng(200 + bits)
    x = rng.standard_normal((20000, D))
    x /= np.linalg.norm(x, axis=1)[:, None]
    q = quantize(x, p["R_eff"], c, t, None)
    xh = dequantize(q, p["R_eff"], c, None)
    mse = np.mean(np.sum((x - xh) ** 2, axis=1))
    assert -0.04 <= mse / Db - 1 <= 0.01


def test_pipeline_takes_the_mode():
    o = Oracle(2, 1, 3, seed=0, rotation="hadamard")
    np.testing.assert_array_equal(o.R_eff, build_params(0, rotation="hadamard")["R_eff"])
