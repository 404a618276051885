"""Whole-path oracle for one preset: parameters, quantize K/V, packed cache, attention.

Ties together lloyd_max, params, quantize, layout and attention for the tests and the
CPU baseline.  Keys use (k_bits, k_qjl); values use v_bits; one seed fixes the
rotation and the sketch (page "Когда в марте 2026 года Google опубликовала статью...":
the codebook is computed once and stored, the method needs no calibration data).
"""
from __future__ import annotations

import math

import numpy as np

from . import layout
from .attention import attend, attend_prefill, key_scores
from .lloyd_max import codebook_f32
from .params import build_params
from .quantize import quantize


class Oracle:
    def __init__(self, k_bits: int, k_qjl: int, v_bits: int, seed: int = 0, d: int = 128, rotation: str = "haar"):
        if k_bits == 0 and not k_qjl:
            raise ValueError("keys need a scalar code or the sign sketch")
        self.k_bits, self.k_qjl, self.v_bits, self.seed, self.d = k_bits, k_qjl, v_bits, seed, d
        self.rotation = rotation
        self.params = build_params(seed, d, rotation=rotation)
        self.R_eff = self.params["R_eff"]
        self.S_b = self.params["S_b"] if k_qjl else None
        if k_bits > 0:
            self.kc, self.kt, self.k_mse = codebook_f32(k_bits)
        else:
            self.kc, self.kt, self.k_mse = None, None, 0.0
        self.vc, self.vt, self.v_mse = codebook_f32(v_bits)

    # ---- quantize-on-write -------------------------------------------------
    def quantize_keys(self, x, force_idx=None, force_mask=None):
        return quantize(x, self.R_eff, self.kc, self.kt, self.S_b, force_idx, force_mask)

    def quantize_values(self, x):
        return quantize(x, self.R_eff, self.vc, self.vt, None)

    # ---- packed cache of one (batch row, kv-head) -------------------------
    def pack_keys(self, kq):
        out = {"n": np.asarray(kq["n"], dtype=np.float32)}
        if self.k_bits > 0:
            out["codes"] = layout.pack(kq["idx"], self.k_bits, "k")
        if self.k_qjl:
            out["signs"] = layout.pack(kq["sign"], 1, "s")
            if self.k_bits > 0:
                out["gamma"] = np.asarray(kq["gamma"], dtype=np.float32)
        return out

    def pack_values(self, vq):
        return {"n": np.asarray(vq["n"], dtype=np.float32), "codes": layout.pack(vq["idx"], self.v_bits, "v")}

    def unpack_keys(self, codes, signs, n, gamma, T):
        k = {"n": np.asarray(n, dtype=np.float32)[:T].astype(np.float64)}
        if self.k_bits > 0:
            k["idx"] = layout.unpack(codes, T, self.d, self.k_bits, "k")
        if self.k_qjl:
            k["sign"] = layout.unpack(signs, T, self.d, 1, "s")
            if self.k_bits > 0:
                k["gamma"] = np.asarray(gamma, dtype=np.float32)[:T].astype(np.float64)
        return k

    def unpack_values(self, codes, n, T):
        return {"n": np.asarray(n, dtype=np.float32)[:T].astype(np.float64),
                "idx": layout.unpack(codes, T, self.d, self.v_bits, "v")}

    # ---- decode attention ---------------------------------------------------
    def attend(self, q, k, v, T=None, scale=None):
        return attend(q, self.R_eff, k, v, self.kc, self.vc, self.S_b, scale=scale, T=T)

    def attend_prefill(self, q, k, v, positions, scale=None):
        return attend_prefill(q, self.R_eff, k, v, self.kc, self.vc, self.S_b, positions, scale=scale)

    def scores(self, q, k):
        return key_scores(q, self.R_eff, k, self.kc, self.S_b) / math.sqrt(self.d)
