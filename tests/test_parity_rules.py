"""CPU checks of the comparison rules the GPU parity tests apply (tests/gpu_harness.py):
the score-magnitude sum used for short rows, the neighbouring-code rule for in-band code
mismatches, and the strict per-row score bound.  Mistakes are planted in oracle output on
the CPU; no GPU is involved."""
import math

import numpy as np
import pytest

from oracle.attention import key_scores
from oracle.pipeline import Oracle
from tests import gpu_harness as H


def _keys(o: Oracle, T, seed):
    rng = np.random.default_rng(seed)
    return o.quantize_keys(rng.standard_normal((T, 128)) * rng.lognormal(0, 0.5, 128))


@pytest.mark.parametrize("preset", [(2, 1, 3), (3, 0, 4), (0, 1, 3)])
def test_score_magnitudes_bound_the_scores(preset):
    o = Oracle(*preset)
    k = _keys(o, 50, 1)
    q = np.random.default_rng(2).standard_normal((4, 128))
    s = key_scores(q, o.R_eff, k, o.kc, o.S_b)
    a = H.score_magnitudes(q, o.R_eff, k, o.kc, o.S_b)
    assert np.all(a >= np.abs(s) * (1 - 1e-12))
    # the bound is not loose by construction: cancellation makes it strictly larger here
    assert np.all(a > np.abs(s))


@pytest.mark.parametrize("preset", [(2, 1, 3), (3, 0, 4), (0, 1, 3)])
def test_score_magnitudes_equal_the_score_when_all_terms_share_a_sign(preset):
    # every term of score i is made non-negative: code j picks a centroid with the sign of
    # q1_j and sign bit j is the sign of q2_j, so the score equals the sum of its magnitudes
    o = Oracle(*preset)
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 128))
    q1 = q @ o.R_eff.T
    T = 5
    k = {"n": rng.uniform(0.5, 2.0, T)}
    if o.kc is not None:
        L = len(o.kc)
        top = rng.integers(L // 2, L, (T, 128))        # positive centroids
        bot = L - 1 - top                               # their mirror images (negative)
        k["idx"] = np.where(q1 >= 0, top, bot).astype(np.uint8)
    if o.S_b is not None:
        q2 = q1 @ o.S_b.T
        k["sign"] = np.repeat(q2 >= 0, T, axis=0)
        if o.kc is not None:
            k["gamma"] = rng.uniform(0.0, 0.3, T)
    s = key_scores(q, o.R_eff, k, o.kc, o.S_b)
    a = H.score_magnitudes(q, o.R_eff, k, o.kc, o.S_b)
    np.testing.assert_allclose(s, a, rtol=1e-12)
    assert np.all(s > 0)


def test_score_magnitudes_scale_with_the_norm_and_ignore_its_sign_flip():
    o = Oracle(2, 1, 3)
    k = _keys(o, 8, 4)
    q = np.random.default_rng(5).standard_normal((2, 128))
    a = H.score_magnitudes(q, o.R_eff, k, o.kc, o.S_b)
    k2 = dict(k, n=3.0 * k["n"])
    np.testing.assert_allclose(H.score_magnitudes(q, o.R_eff, k2, o.kc, o.S_b), 3.0 * a, rtol=1e-14)
    np.testing.assert_allclose(H.score_magnitudes(-q, o.R_eff, k, o.kc, o.S_b), a, rtol=1e-14)


def _quantized_values(seed=6):
    o = Oracle(2, 1, 3)
    x = np.random.default_rng(seed).standard_normal((300, 128))
    return o, o.quantize_values(x)


def test_neighbouring_code_in_band_is_accepted():
    o, ref = _quantized_values()
    got = ref["idx"].copy()
    z = ref["z"].copy()
    # move one coordinate onto threshold t[c] (between codes c and c + 1), and let the GPU
    # side report the other code
    c = 3
    z[10, 7] = o.vt[c] * (1 + 3e-6)
    ref_idx = ref["idx"].copy()
    ref_idx[10, 7] = c + 1
    got[10, 7] = c
    mism, band = H.code_mismatches(got, ref_idx, z, o.vt)
    assert mism.sum() == 1 and band[10, 7]


def test_code_two_steps_away_is_rejected():
    o, ref = _quantized_values()
    z = ref["z"].copy()
    c = 3
    z[10, 7] = o.vt[c] * (1 + 3e-6)
    ref_idx = ref["idx"].copy()
    ref_idx[10, 7] = c + 1
    got = ref_idx.copy()
    got[10, 7] = c - 1  # off by two, though z is in band
    with pytest.raises(AssertionError, match="neighbouring"):
        H.code_mismatches(got, ref_idx, z, o.vt)


def test_neighbour_across_the_wrong_threshold_is_rejected():
    o, ref = _quantized_values()
    z = ref["z"].copy()
    c = 3
    z[10, 7] = o.vt[c] * (1 + 3e-6)  # in the band of t[c] ...
    ref_idx = ref["idx"].copy()
    ref_idx[10, 7] = c
    got = ref_idx.copy()
    got[10, 7] = c - 1  # ... but the codes differ across t[c - 1]
    with pytest.raises(AssertionError, match="threshold between"):
        H.code_mismatches(got, ref_idx, z, o.vt)


def test_mismatch_outside_the_band_is_rejected():
    o, ref = _quantized_values()
    got = ref["idx"].copy()
    i, j = np.argwhere(ref["idx"] == 2)[0]
    got[i, j] = 3
    with pytest.raises(AssertionError):
        H.code_mismatches(got, ref["idx"], ref["z"], o.vt)


def _logits(T=256, H_=4, seed=8):
    o = Oracle(2, 1, 3)
    rng = np.random.default_rng(seed)
    k = o.quantize_keys(rng.standard_normal((T, 128)))
    v = o.quantize_values(rng.standard_normal((T, 128)))
    q = rng.standard_normal((H_, 128))
    logits, _ = o.attend(q, k, v)
    return o, q, k, logits


def test_strict_score_bound_accepts_small_errors_and_rejects_larger_ones():
    o, q, k, logits = _logits()
    rowmax = np.abs(logits).max(axis=1)
    got = logits.copy()
    got[1, 17] += 1.5e-3 * rowmax[1]
    assert H.check_scores(got, logits, logits.shape[1]) == pytest.approx(1.5e-3, rel=1e-9)
    got[2, 200] -= 2.5e-3 * rowmax[2]
    with pytest.raises(AssertionError, match="row maximum"):
        H.check_scores(got, logits, logits.shape[1])


def test_short_rows_use_the_term_magnitudes():
    o, q, k, logits = _logits(T=8)
    mags = H.score_magnitudes(q, o.R_eff, k, o.kc, o.S_b) / math.sqrt(128)
    ref = np.maximum(np.abs(logits).max(axis=1, keepdims=True), mags)
    got = logits + 1.9e-3 * ref
    H.check_scores(got, logits, 8, mags)
    with pytest.raises(AssertionError, match="short row"):
        H.check_scores(logits + 2.1e-3 * ref, logits, 8, mags)


@pytest.mark.parametrize("bits", [1, 3, 4, 6, 8])
def test_threshold_band_tests_the_neighbouring_thresholds_only(bits):
    # the band test looks at the two thresholds around z; written out from its definition
    # (every threshold, one by one) it marks exactly the same elements, including planted
    # values just inside and just outside the bands
    from oracle.lloyd_max import codebook_f32
    from oracle.quantize import threshold_band
    _, t, _ = codebook_f32(bits)
    t64 = t.astype(np.float64)
    rng = np.random.default_rng(bits)
    z = rng.standard_normal((400, 128)) * 1.5
    pick = rng.integers(0, len(t64), 20000)
    z.ravel()[:20000] = t64[pick] * (1 + rng.uniform(-3e-5, 3e-5, 20000)) + rng.uniform(-3e-5, 3e-5, 20000)
    ref = np.zeros(z.shape, dtype=bool)
    for tl in t64:
        ref |= np.abs(z - tl) <= 1e-5 * max(1.0, abs(tl))
    got = threshold_band(z, t)
    np.testing.assert_array_equal(got, ref)
    assert 0 < got.sum() < 20000


def test_sign_band_floor():
    # signs of wide-code keys: the band is 1e-5 max(||r||, ||y|| / 8); a flipped sign whose
    # |u| exceeds it is still rejected, and for 3-bit keys (||r|| > ||y|| / 8) the floor does
    # not widen the band
    o = Oracle(8, 1, 4)
    x = np.random.default_rng(4).standard_normal((64, 128))
    ref = o.quantize_keys(x)
    got = {"n": ref["n"].copy(), "idx": ref["idx"].copy(), "gamma": ref["gamma"].copy(), "sign": ref["sign"].copy()}
    H.compare_keys(o, x, got, {})
    u = ref["u"]
    r_norm = np.linalg.norm(ref["r"], axis=1)
    assert np.all(r_norm < 1 / 8)  # the floor applies to every row
    i, j = np.unravel_index(np.argmin(np.where(np.abs(u) > 2e-5 / 8, np.abs(u), np.inf)), u.shape)
    bad = dict(got, sign=got["sign"].copy())
    bad["sign"][i, j] = not bad["sign"][i, j]
    with pytest.raises(AssertionError, match="sign bit mismatch outside the band"):
        H.compare_keys(o, x, bad, {})
    o3 = Oracle(2, 1, 3)
    r3 = o3.quantize_keys(x)
    assert np.all(np.linalg.norm(r3["r"], axis=1) > 1 / 8)
