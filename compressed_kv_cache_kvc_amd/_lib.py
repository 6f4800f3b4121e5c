"""ctypes declarations of the kvc C ABI (include/kvc.h).  Loading fails loudly
when libkvc.so has not been built: there is no fallback path."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvc.so")

KVC_OK, KVC_ERR_INVALID_ARG, KVC_ERR_UNSUPPORTED, KVC_ERR_WORKSPACE, KVC_ERR_HIP = range(5)
NOALLOC_SCRATCH_BYTES = 64 << 20   # KVC_NOALLOC_SCRATCH_BYTES of include/kvc.h
KVC_F32, KVC_BF16 = 0, 1

# every symbol include/kvc.h declares
EXPORTS = [
    "kvc_fit_assign", "kvc_fit_assign_workspace_bytes",
    "kvc_encode", "kvc_encode_workspace_bytes",
    "kvc_attend", "kvc_attend_workspace_bytes", "kvc_attend_noalloc",
    "kvc_attend_lowdim", "kvc_attend_lowdim_workspace_bytes",
    "kvc_lse_merge", "kvc_assign_qsac", "kvc_query_stats", "kvc_query_stats_workspace_bytes",
    "kvc_route_frames", "kvc_anchor_bits", "kvc_tempo_param_count", "kvc_tempo_encode", "kvc_tempo_decode",
    "kvc_query_moments", "kvc_psac_basis", "kvc_psac_coeffs", "kvc_attend_psac", "kvc_attend_psac_workspace_bytes",
    "kvc_status_string", "kvc_last_error", "kvc_version",
]


class KvcSegment(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("n_centroids", ctypes.c_int32),
        ("rank", ctypes.c_int32),
        ("k_bits", ctypes.c_int32),
        ("v_bits", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("cent_dtype", ctypes.c_int),
        ("k_codes", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("k_meta", ctypes.c_void_p),
        ("v_meta", ctypes.c_void_p),
        ("k_ids", ctypes.c_void_p),
        ("v_ids", ctypes.c_void_p),
        ("k_cent", ctypes.c_void_p),
        ("v_cent", ctypes.c_void_p),
    ]


_i32, _i64, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
_SIGS = {
    "kvc_fit_assign": (ctypes.c_int, [_i32, _i64, _i32, ctypes.c_int, _vp, _i32, _vp, _i32, _vp, _vp, _sz, _vp]),
    "kvc_fit_assign_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32]),
    "kvc_encode": (ctypes.c_int, [_i32, _i64, _i32, ctypes.c_int, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _i32,
                                  _i32, _vp, _vp, _vp, _sz, _vp]),
    "kvc_encode_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32]),
    "kvc_attend": (ctypes.c_int, [_i32, _i64, _i32, ctypes.c_int, _vp, ctypes.POINTER(KvcSegment), _i32, _vp, _vp,
                                  _vp, _sz, _vp]),
    "kvc_attend_workspace_bytes": (_sz, [_i32, _i64, _i32, ctypes.c_int, ctypes.POINTER(KvcSegment), _i32]),
    "kvc_attend_noalloc": (ctypes.c_int, [_i32, _i64, _i32, ctypes.c_int, _vp, ctypes.POINTER(KvcSegment), _i32,
                                          _vp, _vp, _vp]),
    "kvc_attend_lowdim": (ctypes.c_int, [_i32, _i64, _i32, ctypes.c_int, _vp, _vp, _vp, _i32,
                                         ctypes.POINTER(KvcSegment), _i32, _vp, _vp, _vp, _sz, _vp]),
    "kvc_attend_lowdim_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, ctypes.POINTER(KvcSegment), _i32]),
    "kvc_lse_merge": (ctypes.c_int, [_i32, _i64, _i32, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp, _vp,
                                     _vp]),
    "kvc_assign_qsac": (ctypes.c_int, [_i32, _i64, _i32, ctypes.c_int, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp]),
    "kvc_query_stats": (ctypes.c_int, [_i32, _i64, _i32, ctypes.c_int, _vp, _i64, _vp, _vp, _sz, _vp]),
    "kvc_query_stats_workspace_bytes": (_sz, [_i32, _i64, _i32]),
    "kvc_route_frames": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _vp]),
    "kvc_query_moments": (ctypes.c_int, [_i32, _i64, _i32, ctypes.c_int, _vp, _i64, _vp, _vp]),
    "kvc_psac_basis": (ctypes.c_int, [_i32, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp]),
    "kvc_psac_coeffs": (ctypes.c_int, [_i32, _i64, _i32, ctypes.c_int, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _i32,
                                       _vp, _i32, _vp, _vp]),
    "kvc_attend_psac": (ctypes.c_int, [_i32, _i64, _i32, ctypes.c_int, _vp, _vp, _i32, ctypes.POINTER(KvcSegment),
                                       ctypes.POINTER(_vp), _i32, _vp, _vp, _vp, _sz, _vp]),
    "kvc_attend_psac_workspace_bytes": (_sz, [_i32, _i64, _i32, ctypes.c_int, ctypes.POINTER(KvcSegment), _i32]),
    "kvc_anchor_bits": (_i32, [_i32, _i32]),
    "kvc_tempo_param_count": (_i32, [_i32]),
    "kvc_tempo_encode": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, ctypes.c_int, _vp, _vp, _vp, _i32, _i32, _i32,
                                        _vp, _vp, _vp, _vp, _vp, _vp]),
    "kvc_tempo_decode": (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _vp]),
    "kvc_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kvc_last_error": (ctypes.c_char_p, []),
    "kvc_version": (ctypes.c_char_p, []),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libkvc.so (built in-tree by compressed_kv_cache_kvc_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m compressed_kv_cache_kvc_amd.build` "
            "(the HIP kernels are the only implementation; there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
