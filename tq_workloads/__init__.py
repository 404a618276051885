"""Seeded synthetic inputs shared by the oracle tests, the HIP-path tests and the bench.

This module holds no arithmetic of the method: it only draws keys, values and
queries with the shapes and value laws of the workloads, and names the presets.
Every slice (config, batch row b, kv-head h, tensor) is drawn from its own
numpy Generator seeded with [1000 + config index, b, h, tensor id], so any slice
can be regenerated on its own (tensor id 0 = keys, 1 = values, 2 = queries).

Large configurations are drawn on the device with a torch Generator seeded the
same way (``device_slice``); those streams differ from numpy's, and the parity
tests copy the device slices they check back to the host.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

D = 128

# Presets: (k_bits, k_qjl, v_bits).  "turbo3" / "turbo4" are the cache types named on
# the llama.cpp benchmark page ("KV cache benchmark Qwen 3.6-35B-A3B", tables 1-3);
# their bit splits follow the workload definitions (2+1 / 3 and 3+1 / 4).  "turbo2" is the
# 2-bit preset of the fork named in "Когда в марте 2026 года Google опубликовала статью..."
# (paragraph on community implementations), read the same way: 1-bit key code + sign,
# 2-bit values.  "qjl1" keeps
# only the 1-bit sign sketch for keys.  "k8v4" is the asymmetric preset named in the same
# overview's paragraph on K/V asymmetry: 8-bit key codes (no sketch), 4-bit values.
PRESETS = {
    "turbo2": (1, 1, 2),
    "turbo3": (2, 1, 3),
    "turbo4": (3, 1, 4),
    "k8v4": (8, 0, 4),
    "qjl1": (0, 1, 3),
}

TENSOR_K, TENSOR_V, TENSOR_Q = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int            # position in the list of workloads (seeds derive from it)
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int
    dtype: str            # "f32" or "bf16"
    law: str              # "normal" or "student_t"
    nu: float = 0.0       # Student-t degrees of freedom
    n_outlier: int = 0    # outlier channels per (kv-head, tensor)
    outlier_scale: float = 1.0
    lognormal_sigma: float = 0.0   # per-channel scale ~ LogNormal(0, sigma); 0 = none
    presets: tuple = ("turbo3",)
    n_new: int = 0        # new tokens quantized per decode step (per (b, kv-head))

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def cfg_seed(self) -> int:
        return 1000 + self.index


WORKLOADS = [
    Workload(0, "c1_single_head_t4096", B=1, Hq=16, Hkv=1, T=4096, dtype="f32", law="normal",
             n_outlier=4, outlier_scale=8.0, presets=("turbo3",), n_new=1),
    Workload(1, "c2_llama8b_layer_t32k", B=1, Hq=32, Hkv=8, T=32768, dtype="bf16", law="normal",
             lognormal_sigma=0.5, presets=("turbo3", "turbo4"), n_new=1),
    Workload(2, "c3_batch16_t128k", B=16, Hq=32, Hkv=8, T=131072, dtype="bf16", law="student_t",
             nu=5.0, n_outlier=4, outlier_scale=8.0, presets=("turbo3",), n_new=1),
    Workload(3, "c4_llama70b_layer_b8_t128k", B=8, Hq=64, Hkv=8, T=131072, dtype="bf16",
             law="normal", n_outlier=3, outlier_scale=10.0, presets=("qjl1",), n_new=1),
    Workload(4, "c5_moe_attn_t1m", B=1, Hq=32, Hkv=4, T=1048576, dtype="bf16", law="student_t",
             nu=4.0, lognormal_sigma=1.0, presets=("turbo3", "turbo4"), n_new=1),
]


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS:
        if w.name == name_or_index or w.name.startswith(name_or_index + "_"):
            return w
    raise KeyError(name_or_index)


def _rng(w: Workload, b: int, h: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng([w.cfg_seed, b, h, tensor])


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = rounded.astype(np.uint32).view(np.float32)
    # NaN stays NaN (not produced by these generators)
    return out


def channel_scales(w: Workload, h: int, tensor: int, d: int = D) -> np.ndarray:
    """Per-channel multiplier for one (kv-head, tensor): outliers and/or log-normal scales."""
    rng = np.random.default_rng([w.cfg_seed, 0xC4A5, h, tensor])
    s = np.ones(d, dtype=np.float64)
    if w.lognormal_sigma > 0:
        s *= rng.lognormal(0.0, w.lognormal_sigma, size=d)
    if w.n_outlier > 0:
        perm = rng.permutation(d)
        s[perm[: w.n_outlier]] *= w.outlier_scale
    return s


def host_slice(w: Workload, b: int, h: int, tensor: int, t0: int = 0, n: Optional[int] = None,
               d: int = D) -> np.ndarray:
    """Rows [t0, t0+n) of the (b, h, tensor) slice as float32 (bf16-rounded when the workload is bf16).

    Queries (tensor 2) are N(0,1) with one row per q-head of the group (h is the kv-head;
    rows are the G q-heads) and carry no channel scaling.
    """
    rng = _rng(w, b, h, tensor)
    if tensor == TENSOR_Q:
        rows = w.G
        x = rng.standard_normal((rows, d))
    else:
        total = w.T if n is None else t0 + n
        if w.law == "normal":
            x = rng.standard_normal((total, d))
        else:
            x = rng.standard_t(w.nu, size=(total, d))
        x = x[t0:]
        x = x * channel_scales(w, h, tensor, d)[None, :]
    x = x.astype(np.float32)
    if w.dtype == "bf16":
        x = round_to_bf16(x)
    return x


def host_tensor(w: Workload, tensor: int, T: Optional[int] = None, d: int = D) -> np.ndarray:
    """Whole [B, Hkv, T, d] key/value tensor (or [B, Hq, d] queries) on the host, float32."""
    if tensor == TENSOR_Q:
        out = np.empty((w.B, w.Hq, d), dtype=np.float32)
        for b in range(w.B):
            for h in range(w.Hkv):
                out[b, h * w.G:(h + 1) * w.G] = host_slice(w, b, h, TENSOR_Q, d=d)
        return out
    T = w.T if T is None else T
    out = np.empty((w.B, w.Hkv, T, d), dtype=np.float32)
    for b in range(w.B):
        for h in range(w.Hkv):
            out[b, h] = host_slice(w, b, h, tensor, 0, T, d)
    return out


def device_slice(w: Workload, b: int, h: int, tensor: int, T: Optional[int] = None, d: int = D,
                 device="cuda", out=None):
    """Draw one (b, h, tensor) key/value slice [T, d] on the device with a seeded torch Generator.

    Used for the large workloads where drawing on the host would take minutes.  Returns a
    float32 tensor, or writes into ``out`` (bf16 or float32) when given.
    """
    import torch

    T = w.T if T is None else T
    g = torch.Generator(device=device)
    g.manual_seed((w.cfg_seed * 1_000_003 + b * 10_007 + h * 101 + tensor) & 0x7FFFFFFFFFFFFFFF)
    if w.law == "normal":
        x = torch.randn((T, d), generator=g, device=device, dtype=torch.float32)
    else:
        # Student-t(nu) = N(0,1) / sqrt(chi2(nu) / nu); chi2(nu) = 2 * Gamma(nu / 2)
        z = torch.randn((T, d), generator=g, device=device, dtype=torch.float32)
        conc = torch.full((T, d), w.nu / 2.0, device=device, dtype=torch.float32)
        gam = torch._standard_gamma(conc, generator=g)
        x = z / torch.sqrt(2.0 * gam / w.nu)
        del z, conc, gam
    s = torch.from_numpy(channel_scales(w, h, tensor, d).astype(np.float32)).to(device)
    x.mul_(s)
    if out is not None:
        out.copy_(x)
        return out
    if w.dtype == "bf16":
        x = x.to(torch.bfloat16).to(torch.float32)
    return x


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def round_up(a: int, b: int) -> int:
    return ceil_div(a, b) * b


__all__ = [
    "D", "PRESETS", "WORKLOADS", "Workload", "workload", "host_slice", "host_tensor",
    "device_slice", "round_to_bf16", "channel_scales",
    "TENSOR_K", "TENSOR_V", "TENSOR_Q", "ceil_div", "round_up",
]
