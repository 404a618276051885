"""Packed cache layout (oracle side): where every code bit of every token lives.

The pages fix only the size of a block, 52 bytes per 128 values at 3 bits ("Google
TurboQuant простыми словами", section "Бенчмарки TurboQuant", list "Из независимых
реализаций"): 48 bytes of codes plus one 4-byte side value.  The arrangement of the
bits inside the cache is this repo's own and is written out here from its definition,
independently of the HIP code.

Tokens of one (batch row, kv-head) are grouped in blocks of 64.  In block tau, token
p = 64 tau + pp.  A block is split into 64 chunks; chunk L has c = L % 16, g = L // 16.

Key codes (b bits per coordinate, b >= 1), block = 1024 b bytes, chunk = 16 b bytes:
  chunk L holds the 4 tokens pp = 16 t + c (t = 0..3), coordinates j = 32 g + jj
  (jj = 0..31); the code of (t, jj) starts at bit 32 b t + b jj of the chunk.
Key sign bits, block = 1024 bytes, chunk = 16 bytes:
  chunk L holds tokens pp = 16 t + c, sketch rows 32 g + jj; bit 32 t + jj.
Value codes (b bits), block = 1024 b bytes, chunk = 16 b bytes:
  chunk L holds coordinates j = 16 mt + c (mt = 0..7) of the 16 tokens
  pp = 16 t + 4 g + r (t, r = 0..3); the code of (mt, t, r) starts at bit
  4 b (4 mt + t) + b r of the chunk.
Bits are numbered little-endian: bit k of a chunk is bit k % 8 of byte k // 8.
Norms are fp32 arrays in token order, one per (batch row, kv-head, token).
"""
from __future__ import annotations

import numpy as np

BLOCK = 64


def _key_bit_offsets(T: int, d: int, bits: int) -> np.ndarray:
    p = np.arange(T)[:, None]
    j = np.arange(d)[None, :]
    tau, pp = p // BLOCK, p % BLOCK
    t, c = pp // 16, pp % 16
    g, jj = j // 32, j % 32
    L = c + 16 * g
    return tau * (1024 * bits * 8) + L * (128 * bits) + t * (32 * bits) + jj * bits


def _value_bit_offsets(T: int, d: int, bits: int) -> np.ndarray:
    p = np.arange(T)[:, None]
    j = np.arange(d)[None, :]
    tau, pp = p // BLOCK, p % BLOCK
    t, g, r = pp // 16, (pp % 16) // 4, pp % 4
    mt, c = j // 16, j % 16
    L = c + 16 * g
    return tau * (1024 * bits * 8) + L * (128 * bits) + (4 * mt + t) * (4 * bits) + r * bits


def _sign_bit_offsets(T: int, m: int) -> np.ndarray:
    return _key_bit_offsets(T, m, 1)


def _offsets(kind: str, T: int, d: int, bits: int) -> np.ndarray:
    if kind == "k":
        return _key_bit_offsets(T, d, bits)
    if kind == "v":
        return _value_bit_offsets(T, d, bits)
    if kind == "s":
        return _sign_bit_offsets(T, d)
    raise ValueError(kind)


def n_blocks(T: int) -> int:
    return -(-T // BLOCK)


def pack(codes: np.ndarray, bits: int, kind: str) -> np.ndarray:
    """codes [T, d] (ints < 2**bits; bools for kind 's') -> bytes [n_blocks(T), 1024*bits]."""
    codes = np.asarray(codes).astype(np.int64)
    T, d = codes.shape
    bits = 1 if kind == "s" else bits
    nb = n_blocks(T)
    stream = np.zeros(nb * 1024 * bits * 8, dtype=np.uint8)
    off = _offsets(kind, T, d, bits)
    for q in range(bits):
        stream[(off + q).ravel()] = ((codes >> q) & 1).ravel().astype(np.uint8)
    return np.packbits(stream, bitorder="little").reshape(nb, 1024 * bits)


def unpack(packed: np.ndarray, T: int, d: int, bits: int, kind: str) -> np.ndarray:
    """Inverse of pack for the first T tokens: bytes [nb, 1024*bits] -> codes [T, d]."""
    bits = 1 if kind == "s" else bits
    stream = np.unpackbits(np.asarray(packed, dtype=np.uint8).ravel(), bitorder="little")
    off = _offsets(kind, T, d, bits)
    out = np.zeros((T, d), dtype=np.int64)
    for q in range(bits):
        out |= stream[off + q].astype(np.int64) << q
    if kind == "s":
        return out.astype(bool)
    return out.astype(np.uint8)


def block_bytes(bits: int) -> int:
    return 1024 * bits


def bytes_per_token(k_bits: int, k_qjl: int, v_bits: int, d: int = 128) -> dict:
    """Stored bytes per token and kv-head: codes, sign bits and fp32 side values."""
    k = d * k_bits // 8 + (d // 8 if k_qjl else 0) + 4 + (4 if (k_qjl and k_bits > 0) else 0)
    v = d * v_bits // 8 + 4
    return {"k": k, "v": v, "total": k + v}
