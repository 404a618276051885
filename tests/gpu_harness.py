"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI, copy the
packed cache back, and compare it with the oracle under the band rules.

Comparison rules (tolerances of the path):
  * codes: bit-exact, except elements whose rotated value z lies within 1e-5 * max(1, |t|)
    of a threshold t.  A mismatching element must be such an element, the two codes must be
    neighbours (|got - ref| = 1), and z must lie in the band of the one threshold that
    separates them (t[min(got, ref)]); the mismatch fraction must stay below 1e-4 (in-band
    and mismatch fractions are both reported);
  * sign bits: the oracle takes the GPU's code for in-band elements, recomputes the
    residual and its sketch, and must then agree bit for bit except where |u_j| lies
    within 1e-5 * max(||r||, ||y|| / 8) of the decision point 0.  The residual is formed
    from y (unit norm), so its rounding error scales with ||y||, not with ||r||: the floor
    ||y|| / 8 keeps the band above that error for the short residuals of 5..8-bit key codes
    (||r|| ~ 0.05 .. 0.006) and leaves it unchanged for 1..4-bit codes (||r|| >= 0.097);
  * stored norms: relative 1e-6 (vector norms) and 1e-5 (residual norms);
  * scores: per (batch row, q-head), max_i |d score_i| <= 2e-3 max_k |score_k| (the row's
    largest logit).  Only rows of fewer than 64 keys, whose few scores can all nearly
    cancel, fall back to 2e-3 max(max_k |score_k|, A_i) with A_i the sum of the magnitudes
    of the terms of score i (score_magnitudes below);
  * outputs: max |d out| <= 2e-3 max |out| per (batch row, q-head);
    both computed by the oracle on the GPU-written cache.

Every comparison adds its figures to RECORDS; tests/conftest.py prints them at the end of
the run (in-band and mismatch fractions, largest score error against the row maximum,
largest output error).
"""
from __future__ import annotations

import math
import os

import numpy as np

import tq_workloads as wl
from oracle import layout
from oracle.pipeline import Oracle
from oracle.quantize import kappa, sign_band, threshold_band

BAND = 1e-5
SIGN_FLOOR_DIV = 8  # sign band floor: ||y|| / 8
MAX_MISMATCH = 1e-4
SCORE_TOL = 2e-3
# rows with at least this many keys are held to the strict per-row score bound
STRICT_MIN_KEYS = 64

# test id -> {figure: worst value}; printed by tests/conftest.py at the end of the session
RECORDS: dict = {}


def _test_id() -> str:
    cur = os.environ.get("PYTEST_CURRENT_TEST", "interactive")
    return cur.rsplit(" ", 1)[0]


def record(figure: str, value: float, worst=max):
    r = RECORDS.setdefault(_test_id(), {})
    r[figure] = value if figure not in r else worst(r[figure], value)


def torch_mod():
    import torch

    return torch


def to_device(x: np.ndarray, dtype: str, device="cuda"):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def cache_host(cache) -> dict:
    out = {}
    for name, t in cache.tensors().items():
        out[name] = None if t is None else t.cpu().numpy()
    return out


def unpack_keys(orc: Oracle, hc: dict, b: int, h: int, T: int) -> dict:
    k = {"n": hc["k_norm"][b, h, :T].astype(np.float64)}
    if orc.k_bits:
        k["idx"] = layout.unpack(hc["k_codes"][b, h], T, 128, orc.k_bits, "k")
    if orc.k_qjl:
        k["sign"] = layout.unpack(hc["k_signs"][b, h], T, 128, 1, "s")
        if orc.k_bits:
            k["gamma"] = hc["k_rnorm"][b, h, :T].astype(np.float64)
    return k


def unpack_values(orc: Oracle, hc: dict, b: int, h: int, T: int) -> dict:
    return {"n": hc["v_norm"][b, h, :T].astype(np.float64),
            "idx": layout.unpack(hc["v_codes"][b, h], T, 128, orc.v_bits, "v")}


def code_mismatches(got_idx, ref_idx, z, thresholds, rel=BAND):
    """Checks the code rule and returns (mismatch mask, in-band mask).

    Every mismatching element must have codes that are neighbours, and z must lie within
    rel * max(1, |t|) of the threshold t = thresholds[min(got, ref)] that separates them
    (code c covers [t[c-1], t[c]), so t[c] is the boundary between codes c and c + 1)."""
    got = np.asarray(got_idx).astype(np.int64)
    ref = np.asarray(ref_idx).astype(np.int64)
    band = threshold_band(z, thresholds, rel)
    mism = got != ref
    if np.any(mism):
        g, r, zz = got[mism], ref[mism], np.asarray(z, dtype=np.float64)[mism]
        assert np.all(np.abs(g - r) == 1), "a code mismatch is not between neighbouring codes"
        t = np.asarray(thresholds, dtype=np.float32).astype(np.float64)[np.minimum(g, r)]
        assert np.all(np.abs(zz - t) <= rel * np.maximum(1.0, np.abs(t))), \
            "a code mismatch lies outside the band of the threshold between the two codes"
    return mism, band


def compare_keys(orc: Oracle, x: np.ndarray, got: dict, stats: dict):
    """x: the exact input rows [T, d]; got: unpacked GPU keys for the same rows."""
    ref = orc.quantize_keys(x)
    assert np.allclose(got["n"], ref["n"], rtol=1e-6, atol=0), "key norms"
    force = None
    if orc.k_bits:
        mism, band = code_mismatches(got["idx"], ref["idx"], ref["z"], orc.kt)
        _acc(stats, "k_code", mism, band)
        force = (got["idx"], band)
    if orc.k_qjl:
        cond = orc.quantize_keys(x, *force) if force is not None else ref
        y_norm = np.linalg.norm(cond["z"], axis=1) / math.sqrt(cond["z"].shape[1])
        sb = sign_band(cond["u"], np.maximum(np.linalg.norm(cond["r"], axis=1), y_norm / SIGN_FLOOR_DIV), BAND)
        smism = got["sign"] != cond["sign"]
        _acc(stats, "k_sign", smism, sb)
        assert not np.any(smism & ~sb), "sign bit mismatch outside the band"
        if orc.k_bits:
            assert np.allclose(got["gamma"], cond["gamma"], rtol=1e-5, atol=1e-30), "residual norms"
    return ref


def compare_values(orc: Oracle, x: np.ndarray, got: dict, stats: dict):
    ref = orc.quantize_values(x)
    assert np.allclose(got["n"], ref["n"], rtol=1e-6, atol=0), "value norms"
    mism, band = code_mismatches(got["idx"], ref["idx"], ref["z"], orc.vt)
    _acc(stats, "v_code", mism, band)
    return ref


def _acc(stats, key, mism, band):
    s = stats.setdefault(key, {"n": 0, "mismatch": 0, "in_band": 0})
    s["n"] += mism.size
    s["mismatch"] += int(mism.sum())
    s["in_band"] += int(band.sum())


def finish_stats(stats: dict):
    for key, s in stats.items():
        s["mismatch_frac"] = s["mismatch"] / max(1, s["n"])
        s["in_band_frac"] = s["in_band"] / max(1, s["n"])
        record(f"{key}_in_band_frac", s["in_band_frac"])
        record(f"{key}_mismatch_frac", s["mismatch_frac"])
        assert s["mismatch_frac"] < MAX_MISMATCH, (key, s)
    return stats


def score_magnitudes(q, R_eff, k, k_centroids=None, S_b=None):
    """Sum of the magnitudes of the terms of each unscaled score [H, T]:
    n_i (sum_j |q1_j c[idx_ij]| / sqrt(d) + gamma_i kappa sum_j |q2_j|), q1 = R_eff q,
    q2 = S_b q1.  Any finite-precision evaluation of score i errs in proportion to this sum,
    which can be far larger than the score itself when its terms cancel.  Used only for rows
    of fewer than STRICT_MIN_KEYS keys (pinned in tests/test_parity_rules.py)."""
    q = np.asarray(q, dtype=np.float64)
    d = R_eff.shape[0]
    q1 = q @ R_eff.T
    T = len(k["n"])
    acc = np.zeros((q.shape[0], T))
    if k_centroids is not None:
        c = np.asarray(k_centroids, dtype=np.float32).astype(np.float64)
        C = np.abs(c[k["idx"].astype(np.int64)]) / math.sqrt(d)
        acc += np.abs(q1) @ C.T
    if S_b is not None:
        q2 = q1 @ S_b.T
        gamma = k.get("gamma")
        gamma = np.ones(T) if gamma is None else np.asarray(gamma, dtype=np.float64)
        acc += np.abs(q2).sum(axis=1, keepdims=True) * (gamma * kappa(S_b.shape[0]))[None, :]
    return acc * np.abs(np.asarray(k["n"], dtype=np.float64))[None, :]


def check_scores(got, logits, T, mags=None):
    """The score rule on one group of rows: got, logits [H, >= T].  mags (the unscaled-score
    magnitudes times the logit scale) is needed only when T < STRICT_MIN_KEYS.  Returns the
    largest error against each row's largest |logit|."""
    diff = np.abs(np.asarray(got, dtype=np.float64)[:, :T] - logits[:, :T])
    rowmax = np.abs(logits[:, :T]).max(axis=1)
    vs_rowmax = float((diff.max(axis=1) / np.maximum(rowmax, 1e-300)).max())
    if T >= STRICT_MIN_KEYS:
        assert vs_rowmax <= SCORE_TOL, ("scores against the row maximum", vs_rowmax)
    else:
        ref = np.maximum(rowmax[:, None], mags[:, :T])
        assert np.all(diff <= SCORE_TOL * ref), ("scores (short row)", (diff / ref).max())
    return vs_rowmax


def compare_attention(orc: Oracle, q: np.ndarray, k: dict, v: dict, T: int, got_out: np.ndarray,
                      got_scores: np.ndarray = None, scale=None):
    """q [G, d] for one kv-head; k/v unpacked from the GPU cache; got_out [G, d]."""
    logits, out = orc.attend(q.astype(np.float64), k, v, T=T, scale=scale)
    err = {}
    if got_scores is not None:
        mags = None
        if T < STRICT_MIN_KEYS:
            sc = (1.0 / math.sqrt(128)) if scale is None else scale
            kk = {key: np.asarray(val)[:T] for key, val in k.items()}
            mags = sc * score_magnitudes(q.astype(np.float64), orc.R_eff, kk, orc.kc, orc.S_b)
        err["score_vs_rowmax"] = check_scores(got_scores, logits, T, mags)
        record("score_err_vs_rowmax", err["score_vs_rowmax"])
    d = np.abs(got_out - out).max(axis=1)
    ref = np.abs(out).max(axis=1)
    err["out"] = float((d / np.maximum(ref, 1e-300)).max())
    record("out_err_vs_max", err["out"])
    assert np.all(d <= SCORE_TOL * ref), ("outputs", d / ref)
    return err


def make_oracle(preset, seed: int = 0, rotation: str = "haar") -> Oracle:
    """preset: a name of tq_workloads.PRESETS or a (k_bits, k_qjl, v_bits) tuple."""
    return Oracle(*(wl.PRESETS[preset] if isinstance(preset, str) else preset), seed=seed, rotation=rotation)


def hc_inputs_bf16(w: wl.Workload):
    return w.dtype == "bf16"


def relmax(a, b):
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def isqrt_d():
    return 1.0 / math.sqrt(128)
