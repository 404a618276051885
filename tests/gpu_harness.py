"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI, copy the
packed cache back, and compare it with the oracle under the band rules.

Comparison rules (tolerances of the path):
  * codes: bit-exact, except elements whose rotated value z lies within 1e-5 * max(1, |t|)
    of a threshold t; every mismatch must be such an element and the mismatch fraction
    must stay below 1e-4 (in-band and mismatch fractions are both reported);
  * sign bits: the oracle takes the GPU's code for in-band elements, recomputes the
    residual and its sketch, and must then agree bit for bit except where |u_j| lies
    within 1e-5 * ||r|| of the decision point 0;
  * stored norms: relative 1e-6 (vector norms) and 1e-5 (residual norms);
  * scores: |d score_i| <= 2e-3 max(max_k |score_k|, A_i) per (batch row, q-head), where
    A_i is the sum of the magnitudes of the terms of score i (oracle.attention.
    score_magnitudes); A_i only matters when a row's scores all nearly cancel, e.g. a
    single key;
  * outputs: max |d out| <= 2e-3 max |out| per (batch row, q-head);
    both computed by the oracle on the GPU-written cache.
"""
from __future__ import annotations

import math

import numpy as np

import tq_workloads as wl
from oracle import layout
from oracle.pipeline import Oracle
from oracle.attention import score_magnitudes
from oracle.quantize import sign_band, threshold_band

BAND = 1e-5
MAX_MISMATCH = 1e-4
SCORE_TOL = 2e-3


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


def compare_keys(orc: Oracle, x: np.ndarray, got: dict, stats: dict):
    """x: the exact input rows [T, d]; got: unpacked GPU keys for the same rows."""
    ref = orc.quantize_keys(x)
    assert np.allclose(got["n"], ref["n"], rtol=1e-6, atol=0), "key norms"
    force = None
    if orc.k_bits:
        band = threshold_band(ref["z"], orc.kt, BAND)
        mism = got["idx"] != ref["idx"]
        _acc(stats, "k_code", mism, band)
        assert not np.any(mism & ~band), "key code mismatch outside the threshold band"
        force = (got["idx"], band)
    if orc.k_qjl:
        cond = orc.quantize_keys(x, *force) if force is not None else ref
        sb = sign_band(cond["u"], np.linalg.norm(cond["r"], axis=1), BAND)
        smism = got["sign"] != cond["sign"]
        _acc(stats, "k_sign", smism, sb)
        assert not np.any(smism & ~sb), "sign bit mismatch outside the band"
        if orc.k_bits:
            assert np.allclose(got["gamma"], cond["gamma"], rtol=1e-5, atol=1e-30), "residual norms"
    return ref


def compare_values(orc: Oracle, x: np.ndarray, got: dict, stats: dict):
    ref = orc.quantize_values(x)
    assert np.allclose(got["n"], ref["n"], rtol=1e-6, atol=0), "value norms"
    band = threshold_band(ref["z"], orc.vt, BAND)
    mism = got["idx"] != ref["idx"]
    _acc(stats, "v_code", mism, band)
    assert not np.any(mism & ~band), "value code mismatch outside the threshold band"
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
        assert s["mismatch_frac"] < MAX_MISMATCH, (key, s)
    return stats


def compare_attention(orc: Oracle, q: np.ndarray, k: dict, v: dict, T: int, got_out: np.ndarray,
                      got_scores: np.ndarray = None, scale=None):
    """q [G, d] for one kv-head; k/v unpacked from the GPU cache; got_out [G, d]."""
    logits, out = orc.attend(q.astype(np.float64), k, v, T=T, scale=scale)
    err = {}
    if got_scores is not None:
        sc = (1.0 / math.sqrt(128)) if scale is None else scale
        kk = {key: np.asarray(val)[:T] for key, val in k.items()}
        mag = sc * score_magnitudes(q.astype(np.float64), orc.R_eff, kk, orc.kc, orc.S_b)
        ref = np.maximum(np.abs(logits).max(axis=1, keepdims=True), mag)
        rel = np.abs(got_scores[:, :T] - logits) / ref
        err["score"] = float(rel.max())
        err["score_vs_rowmax"] = float((np.abs(got_scores[:, :T] - logits).max(axis=1)
                                        / np.abs(logits).max(axis=1)).max())
        assert np.all(rel <= SCORE_TOL), ("scores", rel.max(axis=1))
    d = np.abs(got_out - out).max(axis=1)
    ref = np.abs(out).max(axis=1)
    err["out"] = float((d / np.maximum(ref, 1e-300)).max())
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
