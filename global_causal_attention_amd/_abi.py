"""ctypes declarations of the C ABI (include/zg_attn.h) and the library loader."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzgattn.so")

ZG_OK, ZG_ERR_NULL, ZG_ERR_SHAPE, ZG_ERR_UNSUPPORTED, ZG_ERR_WORKSPACE, ZG_ERR_HIP = range(6)


class ZgAttnCfg(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("gated", ctypes.c_int32), ("rot_dim", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("rms_eps", ctypes.c_float),
                ("softmax_scale", ctypes.c_float)]


class ZgTokenStrides(ctypes.Structure):
    _fields_ = [("q", ctypes.c_int64), ("k", ctypes.c_int64), ("v", ctypes.c_int64),
                ("gate", ctypes.c_int64), ("out", ctypes.c_int64)]


_P = ctypes.c_void_p
_I32, _I64, _SZ, _F32, _U64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_uint64
_CFG = ctypes.POINTER(ZgAttnCfg)

# name -> (restype, argtypes)
EXPORTS = {
    "zg_attn_prefill_workspace_bytes": (_SZ, [_CFG, _I32, _I32]),
    "zg_attn_prefill": (ctypes.c_int, [_CFG, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P,
                                       ctypes.POINTER(ZgTokenStrides), _P, _P, _SZ, _P]),
    "zg_attn_prefill_cached_workspace_bytes": (_SZ, [_CFG, _I32, _I32]),
    "zg_attn_prefill_cached": (ctypes.c_int, [_CFG, _I32, _I32, _I64, _P, _P, _P, _P, _P, _P,
                                              ctypes.POINTER(ZgTokenStrides), _P, _P, _I64, _P,
                                              _P, _SZ, _P]),
    "zg_attn_decode_workspace_bytes": (_SZ, [_CFG, _I32, _I64]),
    "zg_attn_decode": (ctypes.c_int, [_CFG, _I32, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                      _P, _P, _SZ, _P]),
    "zg_attn_decode_noalloc": (ctypes.c_int, [_CFG, _I32, _I64, _I64, _P, _P, _P, _P, _P, _P,
                                              _P, _P, _P, _P, _P]),
    "zg_attn_decode_fp8": (ctypes.c_int, [_CFG, _I32, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P,
                                          _F32, _F32, _P, _P, _P, _SZ, _P]),
    "zg_kv_to_fp8": (ctypes.c_int, [_P, _P, _I64, _F32, _P]),
    "zg_attn_forward_train_workspace_bytes": (_SZ, [_CFG, _I32, _I32]),
    "zg_attn_forward_train": (ctypes.c_int, [_CFG, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                             _P]),
    "zg_attn_backward_workspace_bytes": (_SZ, [_CFG, _I32, _I32]),
    "zg_attn_backward": (ctypes.c_int, [_CFG, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                        _P, _P, _SZ, _P]),
    "zg_kv_bytes": (_U64, [_I32, _I32, _I32, _I32, _I32, _I32, _I64, _I64]),
    "zg_last_error": (ctypes.c_char_p, []),
    "zg_hbm_read_probe": (ctypes.c_int, [_P, _I64, _P, _I32, _P]),
    "zg_rmsnorm": (ctypes.c_int, [_I64, _I32, _P, _P, _F32, _P, _P]),
    "zg_gemm_bf16": (ctypes.c_int, [_I64, _I32, _I32, _P, _P, _P, _P, _I64, _P]),
    "zg_attn_layer_workspace_bytes": (_SZ, [_CFG, _I32, _I32]),
    "zg_attn_layer": (ctypes.c_int, [_CFG, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "zg_rmsnorm_fp8": (ctypes.c_int, [_I64, _I32, _P, _P, _F32, _P, _P, _P]),
    "zg_quant_rows_fp8": (ctypes.c_int, [_I64, _I32, _P, _I64, _P, _P, _P]),
    "zg_gemm_fp8": (ctypes.c_int, [_I64, _I32, _I32, _P, _P, _P, _P, _P, _P, _I64, _P]),
    "zg_attn_layer_fp8_workspace_bytes": (_SZ, [_CFG, _I32, _I32]),
    "zg_attn_layer_fp8": (ctypes.c_int, [_CFG, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                         _P]),
}

_lib = None


def load_library(path: str | None = None):
    """Load libzgattn.so once. Raises if it is missing: there is no fallback path."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found; build it with `python -m global_causal_attention_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in EXPORTS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib
