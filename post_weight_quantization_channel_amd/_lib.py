"""ctypes loader of libawq.so and the C declarations of include/awq.h.

The library is built in-tree by post_weight_quantization_channel_amd.build. There is no fallback
path: if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libawq.so")

AWQ_OK, AWQ_ERR_NULL, AWQ_ERR_SHAPE, AWQ_ERR_DTYPE, AWQ_ERR_CONFIG, AWQ_ERR_WORKSPACE, \
    AWQ_ERR_HIP = range(7)
AWQ_F32, AWQ_F16, AWQ_BF16 = 0, 1, 2

AWQ_FORM_DIRECT, AWQ_FORM_GRAM = 0, 1

# stage order of awq_search_layer_profiled (the Gram-only stages read 0 in the direct form)
SEARCH_STAGES = ("scale_table", "x_prep", "gram_gemm", "gram_finish", "absmax_w",
                 "quantize_stack", "loss", "finalize")

FLAG_NONFINITE_X = 1 << 0
FLAG_NONFINITE_W = 1 << 1
FLAG_STATS_INEXACT = 1 << 2
FLAG_X_F16_RANGE = 1 << 3
FLAG_SCALE16_OVERFLOW = 1 << 4
FLAG_SCALE16_SUBNORMAL = 1 << 5
FLAG_NONFINITE_LOSS = 1 << 6
FLAG_STEP_UNDERFLOW = 1 << 7
FLAG_CLIP_RANGE = 1 << 8
FLAG_FOLD_RANGE = 1 << 9
FLAG_NO_GRAM = 1 << 10


class AwqCfg(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("n_grid", ctypes.c_int32), ("s_floor", ctypes.c_float), ("form", ctypes.c_int32),
                ("n_clip", ctypes.c_int32), ("clip_min", ctypes.c_float),
                ("zero_point", ctypes.c_int32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t
_E = ctypes.c_int

SIGNATURES = {
    "awq_status_string": (ctypes.c_char_p, [_E]),
    "awq_version": (_I32, []),
    "awq_act_stats_workspace_bytes": (_SZ, [_I64, _I64]),
    "awq_act_stats": (_E, [_P, _E, _I64, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "awq_search_workspace_bytes": (_SZ, [_I64, _I64, _I64, _E, ctypes.POINTER(AwqCfg)]),
    "awq_search_layer": (_E, [_P, _E, _I64, _I64, _P, _E, _I64, _P, ctypes.POINTER(AwqCfg),
                              _P, _P, _P, _P, _P, _SZ, _P]),
    "awq_search_layer_profiled": (_E, [_P, _E, _I64, _I64, _P, _E, _I64, _P,
                                       ctypes.POINTER(AwqCfg), _P, _P, _P, _P, _P, _SZ, _P,
                                       ctypes.POINTER(ctypes.c_float)]),
    "awq_stats_search_layer": (_E, [_P, _E, _I64, _I64, _P, _E, _I64, ctypes.POINTER(AwqCfg),
                                    _P, _P, _P, _P, _P, _P, _SZ, _P,
                                    ctypes.POINTER(ctypes.c_float)]),
    "awq_search_layers": (_E, [ctypes.POINTER(_P), ctypes.POINTER(_I64), _I32, _E, _I64, _P, _E,
                               _I64, _P, ctypes.POINTER(AwqCfg), _P, _P, _P, _P, _P, _SZ, _P]),
    "awq_stats_search_layers": (_E, [ctypes.POINTER(_P), ctypes.POINTER(_I64), _I32, _E, _I64, _P,
                                     _E, _I64, ctypes.POINTER(AwqCfg), _P, _P, _P, _P, _P, _P, _SZ,
                                     _P]),
    "awq_fold_scale": (_E, [_P, _E, _I64, _I64, _I64, _P, _I32, _P, _P]),
    "awq_clip_workspace_bytes": (_SZ, [_I64, _I64, _I64, _E, ctypes.POINTER(AwqCfg)]),
    "awq_clip_search": (_E, [_P, _E, _I64, _I64, _P, _E, _I64, _P, ctypes.POINTER(AwqCfg), _P,
                             _P, _P, _P, _SZ, _P]),
    "awq_clip_search_gram_ws_bytes": (_SZ, [_I64, ctypes.POINTER(AwqCfg)]),
    "awq_clip_search_gram": (_E, [_P, _E, _I64, _I64, _P, ctypes.POINTER(AwqCfg), _P, _SZ, _P,
                                  _P, _P, _P]),
    "awq_pack_int4": (_E, [_P, _E, _I64, _I64, _P, _P, ctypes.POINTER(AwqCfg), _P, _P, _P, _P,
                           _P, _P, _P]),
    "w4a16_gemm": (_E, [_P, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P]),
    "w4a16_gemm_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I32]),
    "w4a16_gemm_ws": (_E, [_P, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "awq_act_stats_noalloc": (_E, [_P, _E, _I64, _I64, _I64, _P, _P, _P]),
}

# bytes of the library's static scratch array (AWQ_NOALLOC_SCRATCH_BYTES in awq.h)
NOALLOC_SCRATCH_BYTES = 32 << 20

_lib = None


def load() -> ctypes.CDLL:
    """Load libawq.so once and attach the C signatures."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m post_weight_quantization_channel_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class AwqError(RuntimeError):
    def __init__(self, call: str, status: int):
        msg = load().awq_status_string(status).decode()
        super().__init__(f"{call}: {msg}")
        self.status = status


def check(call: str, status: int) -> None:
    if status != AWQ_OK:
        raise AwqError(call, status)
