"""ctypes loader for libqasi.so (the gfx950 C-ABI library).

Loading fails loudly when the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqasi.so")

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_i64p = ctypes.POINTER(ctypes.c_int64)

# name -> (restype, argtypes); the exported symbols of include/qasi.h
SIGNATURES = {
    "ts_last_error": (ctypes.c_char_p, []),
    "ts_budget_tokens": (_i64, [_i64, _vp]),
    "ts_score_stride": (_i64, [_i64p, _i32]),
    "ts_index_append": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i32, _vp]),
    "ts_score_workspace_bytes": (_sz, [_i32, _i32]),
    "ts_score": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64p, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "ts_select_workspace_bytes": (_sz, [_i64p, _i32, _i32, _vp]),
    "ts_select": (ctypes.c_int, [_vp, _vp, _i64p, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ts_score_select_workspace_bytes": (_sz, [_i64p, _i32, _i32, _vp]),
    "ts_score_select": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64p, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _sz, _vp]),
    "ts_score_select_state_offset": (_i64, [_i64p, _i32, _i32, _vp]),
    "ts_expand_capacity": (_i64, [_i64, _i64, _i64, _i64, _i64]),
    "ts_expand_workspace_bytes": (_sz, [_i64p, _i32, _i32]),
    "ts_expand_selection": (ctypes.c_int, [_vp, _vp, _i64p, _vp, _i64p, _i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp,
                                           _vp, _sz, _vp]),
    "ts_decode_workspace_bytes": (_sz, [_i64p, _i64p, _i32, _i32, _i32, _i32]),
    "ts_sparse_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64p, _vp, _vp, _i64p, _i32, _i32, _i32, _i32, _vp,
                                        _vp, _sz, _vp]),
    "ts_sparse_decode_timed": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64p, _vp, _vp, _i64p, _i32, _i32, _i32, _i32, _vp,
                                              _vp, _sz, _vp, ctypes.POINTER(ctypes.c_float)]),
    "ts_sparse_decode_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64p, _vp, _vp, _i64p, _i32, _i32, _i32, _i32,
                                                _vp, _vp]),
    "ts_union_workspace_bytes": (_sz, [_i64p, _i32, _i32]),
    "ts_union_lists": (ctypes.c_int, [_vp, _vp, _i64p, _vp, _i64p, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "ts_union_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64p, _vp, _vp, _vp, _vp, _i64p, _i32, _i32, _i32, _vp,
                                       _vp, _sz, _vp]),
    "ts_dense_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64p, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "ts_tiered_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _i64p, _vp, _vp, _i64p, _i32, _i32, _i32,
                                        _i32, _vp, _vp, _sz, _vp]),
    "ts_host_device_pointer": (ctypes.c_int, [_vp, ctypes.POINTER(ctypes.c_void_p)]),
    "snapkv_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i64]),
    "snapkv_compress": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _i32, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _sz, _vp]),
    "snapkv_clusters_workspace_bytes": (_sz, [_i64, _i32]),
    "snapkv_retain_clusters": (ctypes.c_int, [_vp, _i64, _i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                              _vp]),
}


class SelectParams(ctypes.Structure):
    """Mirror of ts_select_params."""
    _fields_ = [("mode", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("budget_num", ctypes.c_int64), ("budget_den", ctypes.c_int64),
                ("sink", ctypes.c_int64), ("local", ctypes.c_int64), ("v_min", ctypes.c_int64),
                ("theta_num", ctypes.c_int64), ("theta_den", ctypes.c_int64)]


_lib = None


def load():
    """Load libqasi.so (raises OSError if it is missing or unloadable)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing: build it first (python -m query_aware_sparse_index_amd.build_lib)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
