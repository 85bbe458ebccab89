"""Loads libfa_mi355x.so and declares the C-ABI signatures of include/fa.h (ctypes).

There is no fallback: if the library is missing the import fails with instructions to build it.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa_mi355x.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python io_aware_attention_fa_amd/build.py` "
        "(or __graft_entry__.build()) first. There is no CPU fallback.")

lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _int, _f32, _size = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                                ctypes.c_size_t)

SIGNATURES = {
    "fa_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _f32, _vp]),
    "fa_fwd_o32": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _f32, _vp]),
    "fa_fwd_strided": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp,
                              _vp, _vp, _int, _f32, _vp]),
    "fa_validate_fwd_strided": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                       _vp, _vp, _vp, _vp, _int, _f32]),
    "fa_decode_workspace_size": (_size, [_i64, _i64, _i64, _i64]),
    "fa_decode": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _i64, _vp, _size,
                         _vp]),
    "fa_decode_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _i64,
                                 _vp]),
    "fa_validate_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _int, _f32]),
    "fa_decode_strided": (_int, [_vp] * 5 + [_i64] * 4 + [_vp] * 4 + [_f32, _i64, _vp, _size,
                                                                       _vp]),
    "fa_validate_decode_strided": (_int, [_vp] * 5 + [_i64] * 4 + [_vp] * 4 + [_f32, _i64, _vp,
                                                                                _size]),
    "fa_validate_decode": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _i64,
                                  _vp, _size]),
    "fa_bwd_workspace_size": (_size, [_i64, _i64, _i64]),
    "fa_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                      _int, _f32, _vp, _size, _vp]),
    "fa_bwd_f32": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                          _i64, _int, _f32, _vp, _size, _vp]),
    "fa_validate_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                               _i64, _i64, _int, _f32, _vp, _size]),
    "fa_bwd_strided": (_int, [_vp] * 9 + [_i64] * 5 + [_vp] * 8 + [_int, _f32, _vp, _size, _vp]),
    "fa_validate_bwd_strided": (_int, [_vp] * 9 + [_i64] * 5 + [_vp] * 8 + [_int, _f32, _vp,
                                                                            _size]),
    "fa_softmax_rows": (_int, [_vp, _vp, _vp, _i64, _i64, _vp]),
    "fa_validate_softmax": (_int, [_vp, _vp, _vp, _i64, _i64]),
    "fa_gelu_f32": (_int, [_vp, _vp, _i64, _vp]),
    "fa_gelu_bf16": (_int, [_vp, _vp, _i64, _vp]),
    "fa_bias_gelu_dropout_bf16": (_int, [_vp, _vp, _vp, _i64, _i64, _f32, ctypes.c_uint64,
                                         ctypes.c_uint64, _vp]),
    "fa_validate_gelu": (_int, [_vp, _vp, _i64]),
    "fa_validate_bias_gelu_dropout": (_int, [_vp, _vp, _vp, _i64, _i64, _f32]),
    "fa_status_str": (ctypes.c_char_p, [_int]),
    "fa_last_hip_error": (_int, []),
}

for _name, (_res, _args) in SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_HEAD_DIM = 3
FA_ERR_CAUSAL_TQ_GT_TK = 4
FA_ERR_ALIGN = 5
FA_ERR_SCALE = 6
FA_ERR_SPLITS = 7
FA_ERR_WORKSPACE = 8
FA_ERR_HIP = 9
FA_ERR_PROB = 10
FA_ERR_SCRATCH = 11
FA_NOALLOC_SCRATCH_BYTES = 33554432   # include/fa.h
