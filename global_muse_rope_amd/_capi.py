"""ctypes declarations of libmuse_attn.so (mirrors include/muse_attn.h)."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# MUSE_ATTN_LIB may name another build of the same library (A/B timing of
# kernel variants); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("MUSE_ATTN_LIB") or os.path.join(_PKG, "libmuse_attn.so")

MUSE_OK = 0
MUSE_ERR_INVALID_ARG = 1
MUSE_ERR_UNSUPPORTED = 2
MUSE_ERR_WORKSPACE = 3
MUSE_ERR_HIP = 4
STATUS_NAMES = {0: "MUSE_OK", 1: "MUSE_ERR_INVALID_ARG", 2: "MUSE_ERR_UNSUPPORTED",
                3: "MUSE_ERR_WORKSPACE", 4: "MUSE_ERR_HIP"}

MUSE_DTYPE_BF16 = 0
MUSE_DTYPE_F16 = 1
MUSE_DTYPE_F32 = 2
MUSE_DTYPE_FP8_E4M3 = 3
MUSE_KV_RING = 0
MUSE_KV_PAGED = 1


class MuseAttnParams(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32),
        ("rope_theta", ctypes.c_float),
        ("qk_scale", ctypes.c_float),
        ("qk_norm_eps", ctypes.c_float),
        ("out_norm", ctypes.c_int32),
        ("out_norm_eps", ctypes.c_float),
    ]


class MuseKvCache(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("max_pages_per_seq", ctypes.c_int32),
        ("page_tokens", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
    ]


class MuseBlockWeights(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("in_norm", ctypes.c_void_p),
        ("w_qkvg", ctypes.c_void_p),
        ("w_o", ctypes.c_void_p),
        ("post_norm", ctypes.c_void_p),
        ("residual_gate", ctypes.c_void_p),
        ("residual_gate_temperature", ctypes.c_float),
    ]


_P = ctypes.POINTER(MuseAttnParams)
_BW = ctypes.POINTER(MuseBlockWeights)
_C = ctypes.POINTER(MuseKvCache)
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

SIGNATURES = {
    "muse_rope_qknorm": (_i32, [_P, _i32, _vp, _i64, _vp, _i64, _vp, _vp, _vp, _i32, _vp]),
    "muse_attn_prefill": (_i32, [_P, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "muse_attn_prefill_workspace_size": (_sz, [_P, _i32, _i32]),
    "muse_attn_prefill_chunk": (_i32, [_P, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _C, _vp, _vp, _sz, _vp]),
    "muse_attn_prefill_chunk_workspace_size": (_sz, [_P, _i32, _i32, _i32]),
    "muse_attn_draft_block": (_i32, [_P, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _C, _vp, _vp, _sz, _vp]),
    "muse_attn_draft_block_workspace_size": (_sz, [_P, _i32, _i32, _i32]),
    "muse_attn_decode": (_i32, [_P, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _C, _vp, _vp, _sz, _vp]),
    "muse_attn_decode_workspace_size": (_sz, [_P, _i32, _i32, _C]),
    "muse_attn_decode_noalloc": (_i32, [_P, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _C, _vp, _vp]),
    "muse_attn_block_prefill": (_i32, [_P, _BW, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "muse_attn_block_prefill_workspace_size": (_sz, [_P, _BW, _i32, _i32]),
    "muse_attn_block_decode": (_i32, [_P, _BW, _i32, _vp, _vp, _i32, _C, _vp, _vp, _sz, _vp]),
    "muse_attn_block_decode_workspace_size": (_sz, [_P, _BW, _i32, _i32, _C]),
    "muse_attn_block_tune": (_i32, [_P, _BW, _i32, _vp, _sz, _vp]),
    "muse_layer_is_global": (_i32, [_i32, _i32]),
    "muse_last_error": (ctypes.c_char_p, []),
    "muse_version": (_i32, []),
    "muse_profile_events": (_i32, [_vp, _vp]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m global_muse_rope_amd.build_lib` "
                "(the attention layer has no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class MuseError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != MUSE_OK:
        msg = load().muse_last_error().decode(errors="replace")
        raise MuseError(status, msg)
