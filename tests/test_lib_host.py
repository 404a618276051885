"""CPU tests of libtq's host side: exports, parameter build parity with the oracle, sizes,
and argument checks that fail before any launch (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_vector_tq_amd as tq
from kv_cache_vector_tq_amd import _lib
from oracle import layout
from oracle.lloyd_max import codebook_f32
from oracle.params import bf16_bits, bf16_value, build_params

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(tq_\w+)\s*\(", text, flags=re.M))
    return names


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert {"tq_build_codebook", "tq_quantize_kv", "tq_attend_decode", "tq_last_error",
            "tq_abi_version", "tq_cache_layout"} <= names
    so = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(so, n), n


def test_abi_version():
    assert tq.tq_abi_version() == 4


@pytest.mark.parametrize("preset", ["turbo2", "turbo3", "turbo4", "qjl1"])
@pytest.mark.parametrize("seed", [0, 1, 12345])
def test_parameter_build_matches_oracle_bit_for_bit(preset, seed):
    kb, kq, vb = tq.PRESETS[preset]
    cb = tq.tq_build_codebook(kb, kq, vb, seed)
    p = build_params(seed)
    np.testing.assert_array_equal(cb.r_hi, p["r_hi"])
    np.testing.assert_array_equal(cb.r_lo, p["r_lo"])
    np.testing.assert_array_equal(cb.rt_hi, p["r_hi"].T)
    np.testing.assert_array_equal(cb.rt_lo, p["r_lo"].T)
    np.testing.assert_array_equal(cb.s_qjl, p["s_b"])
    # M = S_b R_eff as a bf16 pair: hi is M rounded to bf16, and hi + lo is within 2^-16 |M|
    # (two bf16 terms of 8 significant bits each)
    M = p["S_b"] @ p["R_eff"]
    np.testing.assert_array_equal(cb.m_hi, bf16_bits(M))
    pair = bf16_value(cb.m_hi) + bf16_value(cb.m_lo)
    assert np.all(np.abs(pair - M) <= 2.0 ** -16 * np.abs(M) + 1e-30)
    vc, vt, vmse = codebook_f32(vb)
    np.testing.assert_array_equal(cb.v_centroids(), vc)
    np.testing.assert_array_equal(cb.v_thresholds(), vt)
    assert abs(cb.cb.v_mse - vmse) < 1e-15
    if kb:
        kc, kt, kmse = codebook_f32(kb)
        np.testing.assert_array_equal(cb.k_centroids(), kc)
        np.testing.assert_array_equal(cb.k_thresholds(), kt)
        assert abs(cb.cb.k_mse - kmse) < 1e-15


@pytest.mark.parametrize("k_bits", [5, 6, 7, 8])
def test_wide_key_tables_match_oracle_bit_for_bit(k_bits):
    # 5..8-bit key tables: the library's Lloyd iteration with its Newton finish gives the
    # oracle's fp32 tables exactly; entries past 2^b levels stay zero
    cb = tq.tq_build_codebook(k_bits, k_bits % 2, 4, 0)
    kc, kt, kmse = codebook_f32(k_bits)
    np.testing.assert_array_equal(cb.k_centroids(), kc)
    np.testing.assert_array_equal(cb.k_thresholds(), kt)
    assert abs(cb.cb.k_mse - kmse) < 1e-15
    L = 1 << k_bits
    assert not np.any(np.array(cb.cb.k_centroids[L:])) and not np.any(np.array(cb.cb.k_thresholds[L - 1:]))
    with pytest.raises(tq.TQError):
        tq.tq_build_codebook(9, 0, 4, 0)


@pytest.mark.parametrize("preset", ["turbo3", "qjl1"])
@pytest.mark.parametrize("seed", [0, 9])
def test_hadamard_parameter_build_matches_oracle_bit_for_bit(preset, seed):
    kb, kq, vb = tq.PRESETS[preset]
    cb = tq.tq_build_codebook(kb, kq, vb, seed, rotation="hadamard")
    p = build_params(seed, rotation="hadamard")
    np.testing.assert_array_equal(cb.r_hi, p["r_hi"])
    np.testing.assert_array_equal(cb.r_lo, p["r_lo"])
    np.testing.assert_array_equal(cb.rt_hi, p["r_hi"].T)
    np.testing.assert_array_equal(cb.s_qjl, p["s_b"])
    M = p["S_b"] @ p["R_eff"]
    np.testing.assert_array_equal(cb.m_hi, bf16_bits(M))
    assert cb.cb.cfg.rotation == _lib.TQ_ROTATION_HADAMARD


def test_unknown_rotation_rejected():
    cfg = _lib.TQConfig(128, 2, 1, 3, 7, 0)
    cb = _lib.TQCodebook()
    assert _lib.lib.tq_build_codebook(ctypes.byref(cfg), ctypes.byref(cb), None) == _lib.TQ_ERR_UNSUPPORTED
    assert b"rotation" in _lib.lib.tq_last_error()
    with pytest.raises(ValueError):
        tq.tq_build_codebook(2, 1, 3, rotation="dct")


@pytest.mark.parametrize("bad", [dict(k_bits=0, k_qjl=0, v_bits=3), dict(k_bits=9, k_qjl=1, v_bits=3),
                                 dict(k_bits=2, k_qjl=2, v_bits=3), dict(k_bits=2, k_qjl=1, v_bits=0),
                                 dict(k_bits=2, k_qjl=1, v_bits=5)])
def test_bad_configs_rejected(bad):
    with pytest.raises(tq.TQError) as e:
        tq.tq_build_codebook(**bad)
    assert e.value.code == _lib.TQ_ERR_UNSUPPORTED


def test_bad_head_dim_rejected():
    cfg = _lib.TQConfig(64, 2, 1, 3, 0, 0)
    cb = _lib.TQCodebook()
    assert _lib.lib.tq_build_codebook(ctypes.byref(cfg), ctypes.byref(cb), None) == _lib.TQ_ERR_UNSUPPORTED
    assert b"d = 128" in _lib.lib.tq_last_error()
    assert _lib.lib.tq_build_codebook(None, ctypes.byref(cb), None) == _lib.TQ_ERR_INVALID


@pytest.mark.parametrize("preset", ["turbo2", "turbo3", "turbo4", "qjl1"])
def test_cache_layout_sizes(preset):
    kb, kq, vb = tq.PRESETS[preset]
    s = tq.tq_cache_layout(kb, kq, vb, 2, 3, 256)
    slots = 2 * 3 * 256
    assert s["k_codes"] == slots * 128 * kb // 8
    assert s["k_signs"] == (slots * 16 if kq else 0)
    assert s["v_codes"] == slots * 128 * vb // 8
    assert s["k_norm"] == s["v_norm"] == slots * 4
    assert s["bytes_per_token"] == layout.bytes_per_token(kb, kq, vb)["total"]
    with pytest.raises(tq.TQError):
        tq.tq_cache_layout(kb, kq, vb, 1, 1, 100)


class _FakeCache:
    """Cache descriptor with fake (never dereferenced) aligned device addresses."""

    def __init__(self, cb, B=1, Hkv=1, T_cap=64):
        c = cb.cfg
        addr = iter(range(1 << 20, 1 << 30, 1 << 16))
        self.struct = _lib.TQKVCache(next(addr) if c.k_bits else 0, next(addr) if c.k_qjl else 0, next(addr),
                                     next(addr) if (c.k_qjl and c.k_bits) else 0, next(addr), next(addr),
                                     B, Hkv, T_cap)


def _quantize_rc(cb, cache, **kw):
    args = dict(k=1 << 12, v=1 << 13, dtype=_lib.TQ_DTYPE_BF16, B=1, Hkv=1, n_new=1, sb=128, sh=128, st=128,
                start=1 << 14)
    args.update(kw)
    params = _lib.TQDevParams(1 << 15, 1 << 16, 1 << 17, 1 << 18, 1 << 19, 1 << 20, 1 << 21)
    return _lib.lib.tq_quantize_kv(ctypes.byref(cb.cb), ctypes.byref(params), args["k"], args["v"], args["dtype"],
                                   args["B"], args["Hkv"], args["n_new"], args["sb"], args["sh"], args["st"],
                                   args["start"], ctypes.byref(cache.struct), None)


@pytest.mark.parametrize("kw", [dict(k=None, v=None), dict(B=2), dict(n_new=0), dict(st=100), dict(k=(1 << 12) + 2),
                                dict(start=None), dict(sb=-128)])
def test_quantize_argument_checks(kw):
    cb = tq.tq_build_codebook(2, 1, 3)
    assert _quantize_rc(cb, _FakeCache(cb), **kw) == _lib.TQ_ERR_INVALID


def test_quantize_rejects_bad_cache():
    cb = tq.tq_build_codebook(2, 1, 3)
    cache = _FakeCache(cb)
    cache.struct.k_signs = 0
    assert _quantize_rc(cb, cache) == _lib.TQ_ERR_INVALID
    cache = _FakeCache(cb)
    cache.struct.v_codes += 4
    assert _quantize_rc(cb, cache) == _lib.TQ_ERR_INVALID
    cache = _FakeCache(cb, T_cap=100)
    assert _quantize_rc(cb, cache) == _lib.TQ_ERR_INVALID


def _attend_rc(cb, cache, Hq=4, max_seq=64, ws=None, ws_bytes=None, params=None):
    n = ctypes.c_size_t(0 if ws_bytes is None else ws_bytes)
    if params is None:
        params = _lib.TQDevParams(1 << 15, 1 << 16, 1 << 17, 1 << 18, 1 << 19, 1 << 20, 1 << 21)
    rc = _lib.lib.tq_attend_decode(ctypes.byref(cb.cb), ctypes.byref(params), ctypes.byref(cache.struct), 1 << 12,
                                   _lib.TQ_DTYPE_F32, Hq, 1 << 13, max_seq, 0.0, 1 << 14, None, ws, ctypes.byref(n),
                                   None)
    return rc, n.value


def test_attend_workspace_query_and_checks():
    cb = tq.tq_build_codebook(2, 1, 3)
    cache = _FakeCache(cb, B=2, Hkv=2, T_cap=4096)
    rc, need = _attend_rc(cb, cache, Hq=8, max_seq=4096)
    assert rc == _lib.TQ_OK and need > 0
    rc, need2 = _attend_rc(cb, cache, Hq=8, max_seq=4096, ws=1 << 20, ws_bytes=need - 1)
    assert rc == _lib.TQ_ERR_WORKSPACE and need2 == need
    assert _attend_rc(cb, cache, Hq=7)[0] == _lib.TQ_ERR_INVALID          # not a multiple of Hkv
    assert _attend_rc(cb, cache, Hq=2 * 3)[0] == _lib.TQ_ERR_UNSUPPORTED  # group of 3
    assert _attend_rc(cb, cache, Hq=8, max_seq=0)[0] == _lib.TQ_ERR_INVALID
    assert _attend_rc(cb, cache, Hq=8, max_seq=4097)[0] == _lib.TQ_ERR_INVALID
    # the transposed rotation halves are required
    no_rt = _lib.TQDevParams(1 << 15, 1 << 16, 1 << 17, None, 1 << 19, 1 << 20, 1 << 21)
    assert _attend_rc(cb, cache, Hq=8, max_seq=4096, params=no_rt)[0] == _lib.TQ_ERR_INVALID


def _step_rc(cb, cache, k=1 << 12, v=1 << 13, ws=None, ws_bytes=None, Hq=8, start=1 << 14, sb=128, sh=128):
    n = ctypes.c_size_t(0 if ws_bytes is None else ws_bytes)
    params = _lib.TQDevParams(1 << 15, 1 << 16, 1 << 17, 1 << 18, 1 << 19, 1 << 20, 1 << 21)
    rc = _lib.lib.tq_decode_step(ctypes.byref(cb.cb), ctypes.byref(params), ctypes.byref(cache.struct), k, v,
                                 _lib.TQ_DTYPE_BF16, sb, sh, start, 1 << 22, _lib.TQ_DTYPE_BF16, Hq, 1 << 23, 4096,
                                 0.0, 1 << 24, None, ws, ctypes.byref(n), None)
    return rc, n.value


def test_decode_step_checks_before_any_launch():
    cb = tq.tq_build_codebook(2, 1, 3)
    cache = _FakeCache(cb, B=2, Hkv=2, T_cap=4096)
    # workspace query: the attention workspace, nothing launched
    rc, need = _step_rc(cb, cache)
    assert rc == _lib.TQ_OK and need == _attend_rc(cb, cache, Hq=8, max_seq=4096)[1]
    # append errors of tq_quantize_kv, detected on the host with a valid workspace
    assert _step_rc(cb, cache, k=None, v=None, ws=1 << 20, ws_bytes=need)[0] == _lib.TQ_ERR_INVALID
    assert _step_rc(cb, cache, k=(1 << 12) + 2, ws=1 << 20, ws_bytes=need)[0] == _lib.TQ_ERR_INVALID
    assert _step_rc(cb, cache, start=None, ws=1 << 20, ws_bytes=need)[0] == _lib.TQ_ERR_INVALID
    assert _step_rc(cb, cache, sb=-128, ws=1 << 20, ws_bytes=need)[0] == _lib.TQ_ERR_INVALID
    # attention errors come first
    assert _step_rc(cb, cache, Hq=6, ws=1 << 20, ws_bytes=need)[0] == _lib.TQ_ERR_UNSUPPORTED
    assert _step_rc(cb, cache, ws=1 << 20, ws_bytes=need - 1)[0] == _lib.TQ_ERR_WORKSPACE


def test_bf16_baseline_checks():
    n = ctypes.c_size_t(0)
    a = [1 << 12, 1 << 13, 2, 2, 2048, 1 << 14, 8, 1 << 15, 2048, 0.0, 1 << 16]
    assert _lib.lib.tq_bf16_attend_decode(*a, None, ctypes.byref(n), None) == _lib.TQ_OK and n.value > 0
    bad_tcap = list(a)
    bad_tcap[4] = 100
    assert _lib.lib.tq_bf16_attend_decode(*bad_tcap, None, ctypes.byref(n), None) == _lib.TQ_ERR_INVALID
    bad_g = list(a)
    bad_g[6] = 6
    assert _lib.lib.tq_bf16_attend_decode(*bad_g, None, ctypes.byref(n), None) == _lib.TQ_ERR_UNSUPPORTED
    need = n.value
    small = ctypes.c_size_t(need - 1)
    assert _lib.lib.tq_bf16_attend_decode(*a, 1 << 20, ctypes.byref(small), None) == _lib.TQ_ERR_WORKSPACE



def _prefill_rc(cb, cache, q=1 << 12, Hq=8, T_q=100, start=1 << 13, max_seq=4096, out=1 << 14, dtype=None,
                params=None):
    if params is None:
        params = _lib.TQDevParams(1 << 15, 1 << 16, 1 << 17, 1 << 18, 1 << 19, 1 << 20, 1 << 21)
    return _lib.lib.tq_attend_prefill(ctypes.byref(cb.cb), ctypes.byref(params), ctypes.byref(cache.struct), q,
                                      _lib.TQ_DTYPE_BF16 if dtype is None else dtype, Hq, T_q, start, max_seq, 0.0,
                                      out, None)


def test_prefill_argument_checks():
    """Every argument error of tq_attend_prefill is detected on the host (no launch)."""
    cb = tq.tq_build_codebook(2, 1, 3)
    cache = _FakeCache(cb, B=2, Hkv=2, T_cap=4096)
    assert _prefill_rc(cb, cache, q=None) == _lib.TQ_ERR_INVALID
    assert _prefill_rc(cb, cache, start=None) == _lib.TQ_ERR_INVALID
    assert _prefill_rc(cb, cache, out=None) == _lib.TQ_ERR_INVALID
    assert _prefill_rc(cb, cache, q=(1 << 12) + 8) == _lib.TQ_ERR_INVALID     # q not 16-byte aligned
    assert _prefill_rc(cb, cache, out=(1 << 14) + 2) == _lib.TQ_ERR_INVALID   # out not 4-byte aligned
    assert _prefill_rc(cb, cache, T_q=0) == _lib.TQ_ERR_INVALID
    assert _prefill_rc(cb, cache, Hq=7) == _lib.TQ_ERR_INVALID                # not a multiple of Hkv
    assert _prefill_rc(cb, cache, Hq=6) == _lib.TQ_ERR_UNSUPPORTED            # group of 3
    assert _prefill_rc(cb, cache, max_seq=0) == _lib.TQ_ERR_INVALID
    assert _prefill_rc(cb, cache, max_seq=4097) == _lib.TQ_ERR_INVALID
    assert _prefill_rc(cb, cache, dtype=7) == _lib.TQ_ERR_UNSUPPORTED
    no_m = _lib.TQDevParams(1 << 15, 1 << 16, 1 << 17, 1 << 18, 1 << 19, None, 1 << 21)
    assert _prefill_rc(cb, cache, params=no_m) == _lib.TQ_ERR_INVALID         # sketch keys need M
    assert tq.TQError  # the binding raises on these codes
