"""ctypes view of libtis.so: the C-ABI declared in include/tis.h.

Argument marshalling only.  The library must be built (see ``_build``); when
it is missing, loading raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtis.so")

TIS_OK, TIS_E_NULL, TIS_E_SHAPE, TIS_E_DTYPE, TIS_E_ALIGN, TIS_E_UNSUPPORTED, \
    TIS_E_WORKSPACE, TIS_E_HIP = range(8)
TIS_F32, TIS_BF16, TIS_FP8_E4M3 = 0, 1, 2
TIS_MAX_CANDIDATES = 256

STATUS_NAMES = {
    TIS_OK: "TIS_OK", TIS_E_NULL: "TIS_E_NULL", TIS_E_SHAPE: "TIS_E_SHAPE",
    TIS_E_DTYPE: "TIS_E_DTYPE", TIS_E_ALIGN: "TIS_E_ALIGN",
    TIS_E_UNSUPPORTED: "TIS_E_UNSUPPORTED", TIS_E_WORKSPACE: "TIS_E_WORKSPACE",
    TIS_E_HIP: "TIS_E_HIP",
}

TIS_MAX_SURVIVORS = 2048
TIS_NOALLOC_SCRATCH_BYTES = 1 << 20


class TisTree(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("n_keys", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("branching", ctypes.c_int32), ("leaf_block", ctypes.c_int32),
                ("levels", ctypes.c_int32), ("summary_dtype", ctypes.c_int32),
                ("summaries", ctypes.c_void_p)]


class TisCacheTree(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("branching", ctypes.c_int32),
                ("leaf_block", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("n_keys", ctypes.c_int32), ("levels", ctypes.c_int32),
                ("summary_dtype", ctypes.c_int32), ("state_half", ctypes.c_int32),
                ("summaries", ctypes.c_void_p), ("state", ctypes.c_void_p)]


class TisError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_c_int, _c_size, _vp, _c_float = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float

SIGNATURES = {
    "tis_tree_summary_bytes": (_c_size, [_c_int] * 5),
    "tis_tree_summary_bytes_as": (_c_size, [_c_int] * 6),
    "tis_build_workspace_bytes": (_c_size, [_c_int] * 7),
    "tis_tree_build": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                _c_int, ctypes.POINTER(TisTree), _vp, _c_size, _vp]),
    "tis_tree_route": (_c_int, [_vp, _c_int, _c_int, ctypes.POINTER(TisTree), _c_int, _vp, _vp,
                                _vp]),
    "tis_attend_workspace_bytes": (_c_size, [_c_int] * 5),
    "tis_tree_attend": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_int, _vp, _c_int, _c_float, _vp, _vp, _c_size, _vp]),
    "tis_attend_grouped_workspace_bytes": (_c_size, [_c_int] * 5),
    "tis_tree_attend_grouped": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                         _c_int, _c_int, _vp, _c_int, _c_float, _vp, _vp, _c_size,
                                         _vp]),
    "tis_tree_decode": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, ctypes.POINTER(TisTree), _c_int,
                                 _c_float, _vp, _vp, _vp, _c_size, _vp]),
    "tis_decode_workspace_bytes": (_c_size, [_c_int] * 5),
    "tis_tree_decode_noalloc": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, ctypes.POINTER(TisTree),
                                         _c_int, _c_float, _vp, _vp, _vp]),
    "tis_cache_tree_summary_bytes": (_c_size, [_c_int] * 6),
    "tis_cache_tree_summary_bytes_as": (_c_size, [_c_int] * 7),
    "tis_cache_tree_state_bytes": (_c_size, [_c_int] * 6),
    "tis_cache_tree_reset": (_c_int, [ctypes.POINTER(TisCacheTree), _vp]),
    "tis_cache_tree_append": (_c_int, [_vp, _c_int, _c_int, ctypes.POINTER(TisCacheTree), _vp]),
    "tis_cache_tree_route": (_c_int, [_vp, _c_int, _c_int, ctypes.POINTER(TisCacheTree), _c_int,
                                      _vp, _vp, _vp]),
    "tis_cache_tree_decode": (_c_int, [_vp, _vp, _vp, _c_int, _c_int,
                                       ctypes.POINTER(TisCacheTree), _c_int, _c_float, _vp, _vp,
                                       _vp, _c_size, _vp]),
    "tis_cache_tree_append_decode": (_c_int, [_vp, _vp, _vp, _c_int, _c_int,
                                              ctypes.POINTER(TisCacheTree), _c_int, _c_float, _vp,
                                              _vp, _vp, _c_size, _vp]),
    "tis_tree_radius_bytes": (_c_size, [_c_int] * 4),
    "tis_radius_workspace_bytes": (_c_size, [_c_int] * 4),
    "tis_tree_radii": (_c_int, [_vp, _c_int, ctypes.POINTER(TisTree), _vp, _vp, _c_size, _vp]),
    "tis_tree_route_threshold": (_c_int, [_vp, _c_int, _c_int, ctypes.POINTER(TisTree), _vp, _vp,
                                          _c_int, _vp, _vp, _vp]),
    "tis_decode_threshold_workspace_bytes": (_c_size, [_c_int] * 5),
    "tis_tree_decode_threshold": (_c_int, [_vp, _vp, _vp, _c_int, _c_int,
                                           ctypes.POINTER(TisTree), _vp, _vp, _c_int, _c_float,
                                           _vp, _vp, _vp, _vp, _c_size, _vp]),
    "tis_causal_prefill_workspace_bytes": (_c_size, [_c_int] * 10),
    "tis_causal_prefill": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, ctypes.POINTER(TisCacheTree),
                                    _c_int, _c_float, _vp, _vp, _vp, _c_size, _vp]),
    "tis_probe_read": (_c_int, [_vp, _c_size, _c_int, _vp, _vp]),
    "tis_probe_chase": (_c_int, [_vp, _c_size, ctypes.c_uint32, _c_int, _vp, _vp]),
    "tis_probe_decode_timeline_bytes": (_c_size, [_c_int] * 4),
    "tis_probe_decode_timeline": (_c_int, [_vp, _vp, _vp, _c_int, _c_int,
                                           ctypes.POINTER(TisTree), _c_int, _c_float, _vp, _vp,
                                           _c_size, _vp, _c_size, _vp]),
    "tis_wall_clock_khz": (_c_int, [_c_int]),
    "tis_last_error": (ctypes.c_char_p, []),
    "tis_version": (ctypes.c_char_p, []),
}

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"libtis.so not found at {LIB_PATH}; build it with "
                    "`python -m tree_indexed_sparse_build_amd._build`")
            h = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                f = getattr(h, name)
                f.restype = res
                f.argtypes = args
            _lib = h
        return _lib


def check(status: int) -> None:
    if status != TIS_OK:
        msg = lib().tis_last_error().decode(errors="replace")
        raise TisError(status, msg)
