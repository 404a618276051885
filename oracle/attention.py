"""Decode attention straight from the packed codes (oracle, fp64).

Pages: "Когда в марте 2026 года Google опубликовала статью..." (ai-news.ru): the speed-up
is in attention only, and the 1-bit QJL correction passes through the softmax (whose
exponent amplifies its variance); "KV cache benchmark Qwen 3.6-35B-A3B", section
"Неочевидный совет": decoding over a long context is bound by memory bandwidth, which
is why attention reads the compressed cache directly.  "Google TurboQuant простыми
словами", step 2: the sign sketch keeps the attention scores unbiased.

For q-head h of kv-head g (g = h // G), keys 0..T-1:
  q1 = R_eff q;  q2 = S_b q1
  a_i = sum_j q1_j c[idx_ij] / sqrt(d)            (0 when the keys have no scalar code)
  e_i = sum_j q2_j (2 sigma_ij - 1)
  score_i = n_i (a_i + gamma_i kappa e_i),  kappa = sqrt(pi/2) / m
  logit_i = scale * score_i  (scale = 1/sqrt(d) by default)
  p = softmax(logit)  (maximum subtracted)
  o_rot = sum_i p_i nv_i cv[idxv_i] / sqrt(d);  o = R_eff^T o_rot
Since <R_eff q, w> = <q, R_eff^T w>, this equals exact softmax attention over the
dequantized keys and values (checked in the tests).
"""
from __future__ import annotations

import math

import numpy as np

from .quantize import kappa


def key_scores(q, R_eff, k, k_centroids=None, S_b=None):
    """Unscaled scores [H, T] of queries q [H, d] against T keys.

    k: dict with n [T]; idx [T, d] when k_centroids is given; sign [T, m] and gamma [T]
    when S_b is given (gamma may be absent for keys with no scalar code: taken as 1).
    """
    q = np.asarray(q, dtype=np.float64)
    d = R_eff.shape[0]
    q1 = q @ R_eff.T
    T = len(k["n"])
    acc = np.zeros((q.shape[0], T))
    if k_centroids is not None:
        c = np.asarray(k_centroids, dtype=np.float32).astype(np.float64)
        C = c[k["idx"].astype(np.int64)] / math.sqrt(d)
        acc += q1 @ C.T
    if S_b is not None:
        q2 = q1 @ S_b.T
        pm = np.where(k["sign"], 1.0, -1.0)
        gamma = k.get("gamma")
        gamma = np.ones(T) if gamma is None else np.asarray(gamma, dtype=np.float64)
        acc += (q2 @ pm.T) * (gamma * kappa(S_b.shape[0]))[None, :]
    return acc * np.asarray(k["n"], dtype=np.float64)[None, :]


def attend(q, R_eff, k, v, k_centroids, v_centroids, S_b, scale=None, T=None):
    """Decode attention of queries q [H, d] (all of one kv-head) over the first T keys.

    Returns (logits [H, T], out [H, d]).
    """
    d = R_eff.shape[0]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    T = len(k["n"]) if T is None else T
    kk = {key: np.asarray(val)[:T] for key, val in k.items()}
    logits = scale * key_scores(q, R_eff, kk, k_centroids, S_b)
    mx = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - mx)
    p = w / w.sum(axis=1, keepdims=True)
    cv = np.asarray(v_centroids, dtype=np.float32).astype(np.float64)
    V = np.asarray(v["n"], dtype=np.float64)[:T, None] * cv[np.asarray(v["idx"])[:T].astype(np.int64)] / math.sqrt(d)
    o_rot = p @ V
    return logits, o_rot @ R_eff


def attend_prefill(q, R_eff, k, v, k_centroids, v_centroids, S_b, positions, scale=None):
    """Causal (prefill) attention of a prompt's queries straight from the packed codes.

    Pages: "Когда в марте 2026 года Google опубликовала статью..." (ai-news.ru), paragraph
    "Теперь про цифры" (quantization overhead at prefill) and "Google TurboQuant простыми
    словами", section "Как попробовать TurboQuant прямо сейчас" (prefill throughput with the
    compressed cache): the prompt's keys and values are quantized on write and its queries
    attend the compressed cache.  The plainest reading of attention over a prompt is causal:
    the query at absolute position p attends keys 0..p, with the decode score of each key.

    q          [H, Tq, d] queries (all of one kv-head)
    positions  [Tq] absolute positions of the queries (key i is visible when i <= position)
    Returns (logits [H, Tq, T] with -inf at masked keys, out [H, Tq, d]).
    """
    q = np.asarray(q, dtype=np.float64)
    H, Tq, d = q.shape
    positions = np.asarray(positions, dtype=np.int64)
    T = int(positions.max()) + 1
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    kk = {key: np.asarray(val)[:T] for key, val in k.items()}
    logits = scale * key_scores(q.reshape(H * Tq, d), R_eff, kk, k_centroids, S_b).reshape(H, Tq, T)
    visible = np.arange(T)[None, None, :] <= positions[None, :, None]
    logits = np.where(visible, logits, -np.inf)
    mx = logits.max(axis=2, keepdims=True)
    w = np.exp(logits - mx)
    p = w / w.sum(axis=2, keepdims=True)
    cv = np.asarray(v_centroids, dtype=np.float32).astype(np.float64)
    V = np.asarray(v["n"], dtype=np.float64)[:T, None] * cv[np.asarray(v["idx"])[:T].astype(np.int64)] / math.sqrt(d)
    o_rot = p @ V
    return logits, o_rot @ R_eff
