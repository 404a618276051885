"""TurboQuant compressed KV-cache hot path for MI355X: Python binding of libtq.

The functions here carry the names of the C entry points (include/tq.h) and only
marshal arguments: torch tensors own the device memory and supply the stream; every
step of the path runs in the HIP kernels of libtq.so.  Importing this package fails
if libtq.so has not been built.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from . import _lib
from ._lib import (BLOCK_TOKENS, HEAD_DIM, PARAM_NAMES, ROTATIONS, TQ_DTYPE_BF16, TQ_DTYPE_F32, TQCacheSizes,
                   TQCodebook, TQConfig, TQDevParams, TQError, TQHostParams, TQKVCache, check, lib)

PRESETS = {"turbo2": (1, 1, 2), "turbo3": (2, 1, 3), "turbo4": (3, 1, 4), "qjl1": (0, 1, 3), "k8v4": (8, 0, 4)}

__all__ = [
    "PRESETS", "Codebook", "DeviceParams", "KVCache", "TQError", "tq_build_codebook", "tq_cache_layout",
    "tq_decode_step", "tq_bf16_attend_decode", "bf16_value_chunks", "bf16_attend_workspace_bytes",
    "tq_quantize_kv", "tq_attend_decode", "tq_abi_version", "tq_profile_events", "upload_params",
    "attend_workspace_bytes", "tq_read_probe", "tq_attend_decode_noalloc", "tq_attend_prefill",
]


def tq_abi_version() -> int:
    return lib.tq_abi_version()


def tq_profile_events(attend=None, quant=None):
    """Timing hook: pairs of torch.cuda.Event (start, stop) recorded around the main attention
    kernel and around the quantize kernels by later calls on this thread; None disables."""
    def raw(pair):
        if pair is None:
            return None, None
        return tuple(ctypes.c_void_p(e.cuda_event) for e in pair)

    a0, a1 = raw(attend)
    q0, q1 = raw(quant)
    check(lib.tq_profile_events(a0, a1, q0, q1), "tq_profile_events")


@dataclass
class Codebook:
    """Host result of tq_build_codebook: the C struct plus the bf16 bit patterns of the parameter
    matrices (R_hi, R_lo, S_b, R_hi^T, R_lo^T, M_hi, M_lo; 128 x 128 uint16 each)."""
    cb: TQCodebook
    r_hi: np.ndarray
    r_lo: np.ndarray
    s_qjl: np.ndarray
    rt_hi: np.ndarray
    rt_lo: np.ndarray
    m_hi: np.ndarray
    m_lo: np.ndarray

    @property
    def cfg(self) -> TQConfig:
        return self.cb.cfg

    def k_centroids(self):
        return np.array(self.cb.k_centroids[: 1 << self.cfg.k_bits], dtype=np.float32) if self.cfg.k_bits else None

    def k_thresholds(self):
        return np.array(self.cb.k_thresholds[: (1 << self.cfg.k_bits) - 1], dtype=np.float32) if self.cfg.k_bits else None

    def v_centroids(self):
        return np.array(self.cb.v_centroids[: 1 << self.cfg.v_bits], dtype=np.float32)

    def v_thresholds(self):
        return np.array(self.cb.v_thresholds[: (1 << self.cfg.v_bits) - 1], dtype=np.float32)


def _config(k_bits, k_qjl, v_bits, seed, rotation="haar") -> TQConfig:
    if rotation not in ROTATIONS:
        raise ValueError(f"rotation must be one of {sorted(ROTATIONS)}")
    return TQConfig(HEAD_DIM, int(k_bits), int(k_qjl), int(v_bits), ROTATIONS[rotation], int(seed))


def tq_build_codebook(k_bits: int, k_qjl: int, v_bits: int, seed: int = 0, rotation: str = "haar") -> Codebook:
    """rotation: "haar" (seeded Haar-random orthogonal matrix) or "hadamard" (randomized
    Walsh-Hadamard); see tq_build_codebook in include/tq.h."""
    cfg = _config(k_bits, k_qjl, v_bits, seed, rotation)
    cb = TQCodebook()
    mats = {n: np.zeros((HEAD_DIM, HEAD_DIM), dtype=np.uint16) for n in PARAM_NAMES}
    hp = TQHostParams(*(mats[n].ctypes.data for n in PARAM_NAMES))
    check(lib.tq_build_codebook(ctypes.byref(cfg), ctypes.byref(cb), ctypes.byref(hp)), "tq_build_codebook")
    return Codebook(cb, **mats)


def tq_cache_layout(k_bits: int, k_qjl: int, v_bits: int, B: int, Hkv: int, T_cap: int) -> dict:
    cfg = _config(k_bits, k_qjl, v_bits, 0)
    out = TQCacheSizes()
    check(lib.tq_cache_layout(ctypes.byref(cfg), B, Hkv, T_cap, ctypes.byref(out)), "tq_cache_layout")
    return {name: getattr(out, name) for name, _ in TQCacheSizes._fields_}


class DeviceParams:
    """Device copies (torch int16 storage) of the parameter matrices."""

    def __init__(self, codebook: Codebook, device):
        import torch

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)

        self.mats = {n: up(getattr(codebook, n)) for n in PARAM_NAMES}
        for n, t in self.mats.items():
            setattr(self, n, t)
        self.struct = TQDevParams(*(self.mats[n].data_ptr() for n in PARAM_NAMES))


def upload_params(codebook: Codebook, device="cuda") -> DeviceParams:
    return DeviceParams(codebook, device)


class KVCache:
    """Packed cache tensors for B x Hkv x T_cap slots, allocated with torch on `device`."""

    def __init__(self, codebook: Codebook, B: int, Hkv: int, T_cap: int, device="cuda", zero: bool = True):
        import torch

        c = codebook.cfg
        if T_cap % BLOCK_TOKENS:
            raise ValueError("T_cap must be a multiple of 64")
        sizes = tq_cache_layout(c.k_bits, c.k_qjl, c.v_bits, B, Hkv, T_cap)
        alloc = torch.zeros if zero else torch.empty
        nb = T_cap // BLOCK_TOKENS
        self.B, self.Hkv, self.T_cap = B, Hkv, T_cap
        self.k_codes = alloc((B, Hkv, nb, 1024 * c.k_bits), dtype=torch.uint8, device=device) if c.k_bits else None
        self.k_signs = alloc((B, Hkv, nb, 1024), dtype=torch.uint8, device=device) if c.k_qjl else None
        self.k_norm = alloc((B, Hkv, T_cap), dtype=torch.float32, device=device)
        self.k_rnorm = (alloc((B, Hkv, T_cap), dtype=torch.float32, device=device)
                        if (c.k_qjl and c.k_bits) else None)
        self.v_codes = alloc((B, Hkv, nb, 1024 * c.v_bits), dtype=torch.uint8, device=device)
        self.v_norm = alloc((B, Hkv, T_cap), dtype=torch.float32, device=device)
        self.bytes_per_token = sizes["bytes_per_token"]
        self.struct = TQKVCache(*(0 if t is None else t.data_ptr() for t in
                                  (self.k_codes, self.k_signs, self.k_norm, self.k_rnorm, self.v_codes,
                                   self.v_norm)), B, Hkv, T_cap)

    def tensors(self) -> dict:
        return {n: getattr(self, n) for n in ("k_codes", "k_signs", "k_norm", "k_rnorm", "v_codes", "v_norm")}


def _stream(device):
    import torch

    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return TQ_DTYPE_BF16
    if t.dtype == torch.float32:
        return TQ_DTYPE_F32
    raise TypeError(f"inputs must be bfloat16 or float32, got {t.dtype}")


def tq_quantize_kv(codebook: Codebook, params: DeviceParams, cache: KVCache, k, v, start_pos):
    """Quantize k/v ([B, Hkv, n_new, 128], last dim contiguous; either may be None) into the cache
    at slots start_pos[b] + t (start_pos: int32 device tensor [B])."""
    ref = k if k is not None else v
    if ref is None:
        raise ValueError("k and v are both None")
    if k is not None and v is not None and (k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype):
        raise ValueError("k and v must share shape, strides and dtype")
    if ref.dim() != 4 or ref.shape[-1] != HEAD_DIM or ref.stride(-1) != 1:
        raise ValueError("inputs must be [B, Hkv, n_new, 128] with contiguous rows")
    B, Hkv, n_new, _ = ref.shape
    sb, sh, st, _ = ref.stride()
    check(lib.tq_quantize_kv(ctypes.byref(codebook.cb), ctypes.byref(params.struct),
                             k.data_ptr() if k is not None else None, v.data_ptr() if v is not None else None,
                             _dtype_code(ref), B, Hkv, n_new, sb, sh, st, start_pos.data_ptr(),
                             ctypes.byref(cache.struct), _stream(ref.device)), "tq_quantize_kv")


def attend_workspace_bytes(codebook: Codebook, params: DeviceParams, cache: KVCache, Hq: int,
                           max_seq_len: int) -> int:
    """Bytes of attention workspace (no initial contents needed; reusable across calls)."""
    n = ctypes.c_size_t(0)
    # a workspace query needs no device data; dummy non-NULL pointers satisfy the argument check
    check(lib.tq_attend_decode(ctypes.byref(codebook.cb), ctypes.byref(params.struct), ctypes.byref(cache.struct),
                               ctypes.c_void_p(16), TQ_DTYPE_F32, Hq, ctypes.c_void_p(16), max_seq_len, 0.0,
                               ctypes.c_void_p(16), None, None, ctypes.byref(n), None), "tq_attend_decode")
    return n.value


def tq_attend_decode(codebook: Codebook, params: DeviceParams, cache: KVCache, q, seq_len, max_seq_len: int,
                     scale: float = 0.0, out=None, scores_out=None, workspace=None):
    """One decode step: q [B, Hq, 128] (bf16/fp32, contiguous), seq_len int32 device [B].
    Returns out [B, Hq, 128] fp32.  scores_out (optional) is [B, Hq, T_cap] fp32."""
    import torch

    if q.dim() != 3 or q.shape[-1] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 128] tensor")
    B, Hq, _ = q.shape
    if B != cache.B:
        raise ValueError("q batch does not match the cache")
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    need = attend_workspace_bytes(codebook, params, cache, Hq, max_seq_len)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    n = ctypes.c_size_t(workspace.numel())
    check(lib.tq_attend_decode(ctypes.byref(codebook.cb), ctypes.byref(params.struct), ctypes.byref(cache.struct),
                               q.data_ptr(), _dtype_code(q), Hq, seq_len.data_ptr(), max_seq_len, float(scale),
                               out.data_ptr(), scores_out.data_ptr() if scores_out is not None else None,
                               workspace.data_ptr(), ctypes.byref(n), _stream(q.device)), "tq_attend_decode")
    return out


def tq_attend_decode_noalloc(codebook: Codebook, params: DeviceParams, cache: KVCache, q, seq_len,
                             max_seq_len: int, scale: float = 0.0, out=None, scores_out=None):
    """tq_attend_decode with the library's fixed device scratch as workspace (no allocation
    inside the call; `out` must then be given by callers that cannot allocate)."""
    import torch

    if q.dim() != 3 or q.shape[-1] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 128] tensor")
    B, Hq, _ = q.shape
    if B != cache.B:
        raise ValueError("q batch does not match the cache")
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    check(lib.tq_attend_decode_noalloc(ctypes.byref(codebook.cb), ctypes.byref(params.struct),
                                       ctypes.byref(cache.struct), q.data_ptr(), _dtype_code(q), Hq,
                                       seq_len.data_ptr(), max_seq_len, float(scale), out.data_ptr(),
                                       scores_out.data_ptr() if scores_out is not None else None,
                                       _stream(q.device)), "tq_attend_decode_noalloc")
    return out


def tq_attend_prefill(codebook: Codebook, params: DeviceParams, cache: KVCache, q, q_start, max_seq_len: int,
                      scale: float = 0.0, out=None):
    """Causal prefill attention: q [B, Hq, T_q, 128] (bf16/fp32, contiguous), query t of row b at
    position q_start[b] + t (int32 device tensor [B]) attends keys 0 .. q_start[b] + t of the cache.
    Returns out [B, Hq, T_q, 128] fp32."""
    import torch

    if q.dim() != 4 or q.shape[-1] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, T_q, 128] tensor")
    B, Hq, T_q, _ = q.shape
    if B != cache.B:
        raise ValueError("q batch does not match the cache")
    if out is None:
        out = torch.empty((B, Hq, T_q, HEAD_DIM), dtype=torch.float32, device=q.device)
    check(lib.tq_attend_prefill(ctypes.byref(codebook.cb), ctypes.byref(params.struct), ctypes.byref(cache.struct),
                                q.data_ptr(), _dtype_code(q), Hq, T_q, q_start.data_ptr(), max_seq_len,
                                float(scale), out.data_ptr(), _stream(q.device)), "tq_attend_prefill")
    return out


def tq_decode_step(codebook: Codebook, params: DeviceParams, cache: KVCache, k, v, start_pos, q, seq_len,
                   max_seq_len: int, scale: float = 0.0, out=None, scores_out=None, workspace=None):
    """One layer's decode step: quantize the new token k, v ([B, Hkv, 1, 128], last dim
    contiguous; either may be None) into slots start_pos[b], then attend as tq_attend_decode
    (seq_len counts the new token).  Returns out [B, Hq, 128] fp32."""
    import torch

    ref = k if k is not None else v
    if ref is None:
        raise ValueError("k and v are both None")
    if k is not None and v is not None and (k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype):
        raise ValueError("k and v must share shape, strides and dtype")
    if ref.dim() != 4 or ref.shape[2] != 1 or ref.shape[-1] != HEAD_DIM or ref.stride(-1) != 1:
        raise ValueError("new tokens must be [B, Hkv, 1, 128] with contiguous rows")
    if q.dim() != 3 or q.shape[-1] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, Hq, 128] tensor")
    B, Hq, _ = q.shape
    if B != cache.B:
        raise ValueError("q batch does not match the cache")
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    need = attend_workspace_bytes(codebook, params, cache, Hq, max_seq_len)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    n = ctypes.c_size_t(workspace.numel())
    sb, sh, _, _ = ref.stride()
    check(lib.tq_decode_step(ctypes.byref(codebook.cb), ctypes.byref(params.struct), ctypes.byref(cache.struct),
                             k.data_ptr() if k is not None else None, v.data_ptr() if v is not None else None,
                             _dtype_code(ref), sb, sh, start_pos.data_ptr(), q.data_ptr(), _dtype_code(q), Hq,
                             seq_len.data_ptr(), max_seq_len, float(scale), out.data_ptr(),
                             scores_out.data_ptr() if scores_out is not None else None, workspace.data_ptr(),
                             ctypes.byref(n), _stream(q.device)), "tq_decode_step")
    return out


def bf16_value_chunks(v):
    """V [B, Hkv, T, 128] (T a multiple of 32) -> the transposed chunk layout of
    tq_bf16_attend_decode: [B, Hkv, T/32, 128, 32], slot 8 g + e holding key 16 (e / 4) + 4 g + e % 4."""
    import torch

    B, Hkv, T, _ = v.shape
    order = torch.tensor([16 * (e // 4) + 4 * g + e % 4 for g in range(4) for e in range(8)], device=v.device)
    return v.reshape(B, Hkv, T // 32, 32, HEAD_DIM)[:, :, :, order, :].transpose(3, 4).contiguous()


def bf16_attend_workspace_bytes(B: int, Hkv: int, T_cap: int, Hq: int, max_seq_len: int) -> int:
    """Bytes of workspace tq_bf16_attend_decode needs (no initial contents)."""
    n = ctypes.c_size_t(0)
    # a workspace query needs no device data; dummy aligned pointers satisfy the argument checks
    check(lib.tq_bf16_attend_decode(ctypes.c_void_p(256), ctypes.c_void_p(256), B, Hkv, T_cap, ctypes.c_void_p(256),
                                    Hq, ctypes.c_void_p(256), max_seq_len, 0.0, ctypes.c_void_p(256), None,
                                    ctypes.byref(n), None), "tq_bf16_attend_decode")
    return n.value


def tq_bf16_attend_decode(k, vt, q, seq_len, max_seq_len: int, scale: float = 0.0, out=None, workspace=None):
    """Uncompressed bf16 baseline: k [B, Hkv, T_cap, 128] bf16, vt from bf16_value_chunks(v),
    q [B, Hq, 128] bf16.  Returns out [B, Hq, 128] fp32."""
    import torch

    B, Hkv, T_cap, _ = k.shape
    Hq = q.shape[1]
    if out is None:
        out = torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    need = bf16_attend_workspace_bytes(B, Hkv, T_cap, Hq, max_seq_len)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    n = ctypes.c_size_t(workspace.numel())
    check(lib.tq_bf16_attend_decode(k.data_ptr(), vt.data_ptr(), B, Hkv, T_cap, q.data_ptr(), Hq, seq_len.data_ptr(),
                                    max_seq_len, float(scale), out.data_ptr(), workspace.data_ptr(), ctypes.byref(n),
                                    _stream(q.device)), "tq_bf16_attend_decode")
    return out



def tq_read_probe(buf, grid: int, sink=None):
    """Read-bandwidth probe: one launch reading all of `buf` (a contiguous device tensor whose
    byte size is a multiple of 16) with 16-byte loads on `grid` workgroups of 256 lanes."""
    import torch

    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    check(lib.tq_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), int(grid),
                            _stream(buf.device)), "tq_read_probe")
    return sink
