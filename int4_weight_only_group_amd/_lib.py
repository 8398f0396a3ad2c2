"""ctypes loader for libw4.so (the HIP library).  No fallback: a missing library raises."""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4.so")

# name -> (restype, argtypes); mirrors include/w4.h
_c = ctypes
_i64, _p, _sz_p = _c.c_int64, _c.c_void_p, _c.POINTER(_c.c_size_t)
SIGNATURES = {
    "w4_strerror": (_c.c_char_p, [_c.c_int]),
    "w4_pack": (_c.c_int, [_p, _p, _i64, _i64, _p]),
    "w4_gemv": (_c.c_int, [_p, _p, _p, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _sz_p, _p]),
    "w4_dequant_f16_t": (_c.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "w4_quantize": (_c.c_int, [_p, _i64, _p, _p, _p, _i64, _i64, _p]),
    "w4_gemv_sym128": (_c.c_int, [_p, _p, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _sz_p, _p]),
    "w4_dequant_f16_t_sym128": (_c.c_int, [_p, _p, _p, _i64, _i64, _i64, _p]),
    "gemm_f16": (_c.c_int, [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _sz_p, _p]),
    "gemm_f16_dequant_next": (_c.c_int, [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _sz_p,
                                         _p, _p, _p, _p, _i64, _i64, _i64, _p]),
    "gemm_f16_dequant_next_sym128": (_c.c_int, [_p, _i64, _p, _i64, _p, _i64, _i64, _i64, _i64, _p, _sz_p,
                                                _p, _p, _p, _i64, _i64, _i64, _p]),
    "logits_argmax_topk": (_c.c_int, [_p, _i64, _i64, _i64, _i64, _p, _p, _p, _sz_p, _p]),
    "logits_argmax_topk_noalloc": (_c.c_int, [_p, _i64, _i64, _i64, _i64, _p, _p, _p]),
    "w4_gemv_topk": (_c.c_int, [_p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p, _sz_p, _p]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libw4.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m int4_weight_only_group_amd.build` "
                "(there is no CPU fallback)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib
