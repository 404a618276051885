"""Pins of the decode-attention oracle: dense dequantized attention, special cases."""
import math

import numpy as np
import pytest

from oracle.pipeline import Oracle
from oracle.quantize import dequantize


def _setup(preset, T, G, seed=0):
    k_bits, k_qjl, v_bits = preset
    o = Oracle(k_bits, k_qjl, v_bits, seed=0)
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((T, 128)) * rng.lognormal(0, 0.5, 128)
    V = rng.standard_normal((T, 128))
    Q = rng.standard_normal((G, 128))
    return o, K, V, Q


def _dense(o, Q, kq, vq, scale=None):
    """softmax(q . k~ * scale) V^ with the dequantized vectors in the original domain."""
    Kd = dequantize(kq, o.R_eff, o.kc, o.S_b)
    Vd = dequantize(vq, o.R_eff, o.vc, None)
    scale = 1 / math.sqrt(128) if scale is None else scale
    logits = scale * Q @ Kd.T
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return logits, p @ Vd


@pytest.mark.parametrize("preset", [(2, 1, 3), (3, 1, 4), (0, 1, 3), (2, 0, 3), (8, 0, 4), (5, 1, 3)])
@pytest.mark.parametrize("T", [1, 7, 64])
def test_matches_dense_dequantized_attention(preset, T):
    o, K, V, Q = _setup(preset, T, 4, seed=T)
    kq, vq = o.quantize_keys(K), o.quantize_values(V)
    logits, out = o.attend(Q, kq, vq)
    dl, do = _dense(o, Q, kq, vq)
    np.testing.assert_allclose(logits, dl, rtol=1e-12, atol=1e-12 * np.abs(dl).max())
    np.testing.assert_allclose(out, do, rtol=1e-11, atol=1e-12 * np.abs(do).max())


def test_single_key_returns_its_value():
    o, K, V, Q = _setup((2, 1, 3), 1, 3)
    kq, vq = o.quantize_keys(K), o.quantize_values(V)
    _, out = o.attend(Q, kq, vq)
    vhat = dequantize(vq, o.R_eff, o.vc, None)[0]
    for h in range(3):
        np.testing.assert_allclose(out[h], vhat, rtol=1e-12, atol=1e-13)


def test_zero_query_averages_values():
    o, K, V, Q = _setup((2, 1, 3), 40, 2)
    kq, vq = o.quantize_keys(K), o.quantize_values(V)
    _, out = o.attend(np.zeros((1, 128)), kq, vq)
    vhat = dequantize(vq, o.R_eff, o.vc, None)
    np.testing.assert_allclose(out[0], vhat.mean(axis=0), rtol=1e-12, atol=1e-13)


def test_identical_keys_give_uniform_weights():
    o, K, V, Q = _setup((3, 1, 4), 30, 2)
    K[:] = K[0]
    kq, vq = o.quantize_keys(K), o.quantize_values(V)
    logits, out = o.attend(Q, kq, vq)
    assert np.ptp(logits, axis=1).max() <= 1e-14 * np.abs(logits).max()
    vhat = dequantize(vq, o.R_eff, o.vc, None)
    np.testing.assert_allclose(out, np.repeat(vhat.mean(axis=0)[None], 2, 0), rtol=1e-12, atol=1e-13)


def test_scores_reduce_to_inner_product_without_codes():
    # keys with no scalar code: score = n * kappa * <S q1, 2 sigma - 1>
    o, K, V, Q = _setup((0, 1, 3), 10, 2)
    kq = o.quantize_keys(K)
    s = o.scores(Q, kq) * math.sqrt(128)
    q1 = Q @ o.R_eff.T
    pm = np.where(kq["sign"], 1.0, -1.0)
    ref = (q1 @ o.S_b.T) @ pm.T * (math.sqrt(math.pi / 2) / 128) * kq["n"][None, :]
    np.testing.assert_allclose(s, ref, rtol=1e-12)


def test_packed_cache_round_trip_gives_same_attention():
    o, K, V, Q = _setup((2, 1, 3), 150, 4)
    kq, vq = o.quantize_keys(K), o.quantize_values(V)
    pk, pv = o.pack_keys(kq), o.pack_values(vq)
    k2 = o.unpack_keys(pk["codes"], pk["signs"], pk["n"], pk["gamma"], 150)
    v2 = o.unpack_values(pv["codes"], pv["n"], 150)
    l1, o1 = o.attend(Q, kq, vq)
    l2, o2 = o.attend(Q, k2, v2)
    # only the fp32 storage of the norms differs
    np.testing.assert_allclose(l2, l1, rtol=1e-6, atol=1e-6 * np.abs(l1).max())
    np.testing.assert_allclose(o2, o1, rtol=1e-5, atol=1e-6 * np.abs(o1).max())


@pytest.mark.parametrize("preset,min_corr", [((3, 1, 4), 0.95), ((2, 1, 3), 0.88), ((2, 0, 3), 0.9),
                                               ((8, 0, 4), 0.999), ((6, 1, 4), 0.995)])
def test_logits_track_unquantized_logits(preset, min_corr):
    # Not a pin (the pages give no accuracy figure for a stated workload): a sanity floor
    # on the correlation of the estimated logits with exact fp64 logits on the raw keys.
    o, K, V, Q = _setup(preset, 512, 8, seed=9)
    kq, vq = o.quantize_keys(K), o.quantize_values(V)
    logits, _ = o.attend(Q, kq, vq)
    exact = Q @ K.T / math.sqrt(128)
    corr = [np.corrcoef(logits[h], exact[h])[0, 1] for h in range(8)]
    assert min(corr) > min_corr


# ---- prefill (causal) attention ---------------------------------------------------------------

@pytest.mark.parametrize("preset", [(2, 1, 3), (3, 1, 4), (0, 1, 3), (2, 0, 3)])
def test_prefill_matches_dense_masked_attention(preset):
    # softmax over the visible keys of q . k~ / sqrt(d), written out with an explicit loop over
    # query positions and the dequantized vectors (independent of the vectorized mask)
    o, K, V, Q = _setup(preset, 40, 3, seed=5)
    Qp = np.random.default_rng(6).standard_normal((3, 12, 128))
    positions = np.array([0, 1, 5, 13, 20, 21, 22, 30, 31, 37, 38, 39])
    kq, vq = o.quantize_keys(K), o.quantize_values(V)
    logits, out = o.attend_prefill(Qp, kq, vq, positions)
    Kd = dequantize(kq, o.R_eff, o.kc, o.S_b)
    Vd = dequantize(vq, o.R_eff, o.vc, None)
    for h in range(3):
        for j, pos in enumerate(positions):
            s = Qp[h, j] @ Kd[:pos + 1].T / math.sqrt(128)
            p = np.exp(s - s.max())
            p /= p.sum()
            np.testing.assert_allclose(logits[h, j, :pos + 1], s, rtol=1e-12, atol=1e-12 * np.abs(s).max())
            assert np.all(np.isneginf(logits[h, j, pos + 1:]))
            np.testing.assert_allclose(out[h, j], p @ Vd[:pos + 1], rtol=1e-11, atol=1e-12 * np.abs(out[h, j]).max())


def test_prefill_rows_reduce_to_decode_and_first_value():
    o, K, V, Q = _setup((2, 1, 3), 64, 4, seed=8)
    kq, vq = o.quantize_keys(K), o.quantize_values(V)
    Qp = np.random.default_rng(9).standard_normal((4, 64, 128))
    _, out = o.attend_prefill(Qp, kq, vq, np.arange(64))
    # the last query sees every key: decode attention over all 64 keys
    _, dec = o.attend(Qp[:, -1], kq, vq)
    np.testing.assert_allclose(out[:, -1], dec, rtol=1e-12, atol=1e-13)
    # the first query sees only key 0: its value, whatever the query
    vhat = dequantize(vq, o.R_eff, o.vc, None)[0]
    for h in range(4):
        np.testing.assert_allclose(out[h, 0], vhat, rtol=1e-12, atol=1e-13)
    # a query at position p equals decode attention over keys 0..p
    for p_ in (7, 31, 50):
        _, dp = o.attend(Qp[:, p_], kq, vq, T=p_ + 1)
        np.testing.assert_allclose(out[:, p_], dp, rtol=1e-12, atol=1e-13)
