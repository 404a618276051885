"""ctypes view of libtq (include/tq.h): structures and raw entry points.

Loads the in-tree libtq.so built by build_lib.py.  There is no fallback: if the
library is missing or cannot be loaded, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtq.so")

TQ_OK = 0
TQ_ERR_INVALID = -1
TQ_ERR_UNSUPPORTED = -2
TQ_ERR_WORKSPACE = -3
TQ_ERR_DEVICE = -4
TQ_DTYPE_BF16 = 0
TQ_DTYPE_F32 = 1
HEAD_DIM = 128
MAX_K_LEVELS = 256
BLOCK_TOKENS = 64

ERROR_NAMES = {
    TQ_ERR_INVALID: "TQ_ERR_INVALID",
    TQ_ERR_UNSUPPORTED: "TQ_ERR_UNSUPPORTED",
    TQ_ERR_WORKSPACE: "TQ_ERR_WORKSPACE",
    TQ_ERR_DEVICE: "TQ_ERR_DEVICE",
}


class TQConfig(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("k_bits", ctypes.c_int32), ("k_qjl", ctypes.c_int32),
                ("v_bits", ctypes.c_int32), ("rotation", ctypes.c_int32), ("seed", ctypes.c_uint64)]


TQ_ROTATION_HAAR, TQ_ROTATION_HADAMARD = 0, 1
ROTATIONS = {"haar": TQ_ROTATION_HAAR, "hadamard": TQ_ROTATION_HADAMARD}


class TQCodebook(ctypes.Structure):
    _fields_ = [("cfg", TQConfig),
                ("k_centroids", ctypes.c_float * MAX_K_LEVELS), ("k_thresholds", ctypes.c_float * MAX_K_LEVELS),
                ("v_centroids", ctypes.c_float * 16), ("v_thresholds", ctypes.c_float * 16),
                ("k_mse", ctypes.c_double), ("v_mse", ctypes.c_double)]


class TQDevParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("r_hi", "r_lo", "s_qjl", "rt_hi", "rt_lo", "m_hi", "m_lo")]


class TQHostParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("r_hi", "r_lo", "s_qjl", "rt_hi", "rt_lo", "m_hi", "m_lo")]


PARAM_NAMES = ("r_hi", "r_lo", "s_qjl", "rt_hi", "rt_lo", "m_hi", "m_lo")


class TQKVCache(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_signs", ctypes.c_void_p), ("k_norm", ctypes.c_void_p),
                ("k_rnorm", ctypes.c_void_p), ("v_codes", ctypes.c_void_p), ("v_norm", ctypes.c_void_p),
                ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("T_cap", ctypes.c_int32)]


class TQCacheSizes(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_size_t), ("k_signs", ctypes.c_size_t), ("k_norm", ctypes.c_size_t),
                ("k_rnorm", ctypes.c_size_t), ("v_codes", ctypes.c_size_t), ("v_norm", ctypes.c_size_t),
                ("bytes_per_token", ctypes.c_size_t)]


class TQError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where}: {ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libtq.so is not built ({LIB_PATH}); run kv_cache_vector_tq_amd.build_lib")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.tq_abi_version.restype = ctypes.c_int
    lib.tq_abi_version.argtypes = []
    lib.tq_last_error.restype = ctypes.c_char_p
    lib.tq_last_error.argtypes = []
    lib.tq_build_codebook.restype = ctypes.c_int
    lib.tq_build_codebook.argtypes = [P(TQConfig), P(TQCodebook), P(TQHostParams)]
    lib.tq_cache_layout.restype = ctypes.c_int
    lib.tq_cache_layout.argtypes = [P(TQConfig), ctypes.c_int, ctypes.c_int, ctypes.c_int, P(TQCacheSizes)]
    lib.tq_quantize_kv.restype = ctypes.c_int
    lib.tq_quantize_kv.argtypes = [P(TQCodebook), P(TQDevParams), vp, vp, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   vp, P(TQKVCache), vp]
    lib.tq_attend_decode.restype = ctypes.c_int
    lib.tq_attend_decode.argtypes = [P(TQCodebook), P(TQDevParams), P(TQKVCache), vp, ctypes.c_int,
                                     ctypes.c_int, vp, ctypes.c_int, ctypes.c_float, vp, vp, vp,
                                     P(ctypes.c_size_t), vp]
    lib.tq_attend_decode_noalloc.restype = ctypes.c_int
    lib.tq_attend_decode_noalloc.argtypes = [P(TQCodebook), P(TQDevParams), P(TQKVCache), vp, ctypes.c_int,
                                             ctypes.c_int, vp, ctypes.c_int, ctypes.c_float, vp, vp, vp]
    lib.tq_attend_prefill.restype = ctypes.c_int
    lib.tq_attend_prefill.argtypes = [P(TQCodebook), P(TQDevParams), P(TQKVCache), vp, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, vp, ctypes.c_int, ctypes.c_float, vp, vp]
    lib.tq_decode_step.restype = ctypes.c_int
    lib.tq_decode_step.argtypes = [P(TQCodebook), P(TQDevParams), P(TQKVCache), vp, vp, ctypes.c_int,
                                   ctypes.c_int64, ctypes.c_int64, vp, vp, ctypes.c_int, ctypes.c_int, vp,
                                   ctypes.c_int, ctypes.c_float, vp, vp, vp, P(ctypes.c_size_t), vp]
    lib.tq_bf16_attend_decode.restype = ctypes.c_int
    lib.tq_bf16_attend_decode.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, ctypes.c_int, vp,
                                          ctypes.c_int, ctypes.c_float, vp, vp, P(ctypes.c_size_t), vp]
    lib.tq_read_probe.restype = ctypes.c_int
    lib.tq_read_probe.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_int, vp]
    lib.tq_profile_events.restype = ctypes.c_int
    lib.tq_profile_events.argtypes = [vp, vp, vp, vp]
    return lib


lib = _load()


def check(rc: int, where: str):
    if rc != TQ_OK:
        raise TQError(rc, where, lib.tq_last_error().decode())
    return rc
