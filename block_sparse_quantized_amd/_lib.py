"""ctypes view of libsparge.so: structs and prototypes mirroring include/sparge.h."""

from __future__ import annotations

import ctypes
import os
import threading

SPARGE_F32, SPARGE_F16, SPARGE_BF16 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.environ.get("SPARGE_LIB", os.path.join(_HERE, "libsparge.so"))


class SpargeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class SpargeTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("D", ctypes.c_int64), ("sB", ctypes.c_int64), ("sH", ctypes.c_int64),
                ("sN", ctypes.c_int64)]


class SpargeStats(ctypes.Structure):
    _fields_ = [("valid_blocks", ctypes.c_uint64), ("kept_blocks", ctypes.c_uint64),
                ("group_updates", ctypes.c_uint64), ("skipped_updates", ctypes.c_uint64)]


class SpargeOpts(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_double), ("sim_threshold", ctypes.c_double),
                ("filter_lambda", ctypes.c_double), ("filter_on", ctypes.c_int32),
                ("qk_int8", ctypes.c_int32), ("pv_fp16", ctypes.c_int32),
                ("pv_fp8", ctypes.c_int32), ("mask_out", ctypes.c_void_p),
                ("stats", ctypes.POINTER(SpargeStats)), ("prof_start", ctypes.c_void_p),
                ("prof_attn_begin", ctypes.c_void_p), ("prof_attn_end", ctypes.c_void_p),
                ("head_select", ctypes.POINTER(ctypes.c_double)),
                ("head_sim_threshold", ctypes.POINTER(ctypes.c_double)),
                ("head_filter_lambda", ctypes.POINTER(ctypes.c_double))]


_P = ctypes.POINTER
_T = _P(SpargeTensor)
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64

PROTOTYPES = {
    "sparge_default_opts": (None, [_P(SpargeOpts)]),
    "sparge_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, _i64, _i32, _P(SpargeOpts)]),
    "sparge_topk_attn": (_i32, [_T, _T, _T, _T, ctypes.c_double, _i32, _P(SpargeOpts), _vp,
                                ctypes.c_size_t, _vp]),
    "sparge_cdf_attn": (_i32, [_T, _T, _T, _T, ctypes.c_double, _i32, _P(SpargeOpts), _vp,
                               ctypes.c_size_t, _vp]),
    "sparge_topk_attn_noalloc": (_i32, [_T, _T, _T, _T, ctypes.c_double, _i32, _P(SpargeOpts), _vp]),
    "block_sparse_attn": (_i32, [_T, _T, _T, _vp, _T, _P(SpargeOpts), _vp, ctypes.c_size_t, _vp]),
    "sparge_predict_mask": (_i32, [_T, _T, ctypes.c_double, _i32, _P(SpargeOpts), _vp, _vp,
                                   ctypes.c_size_t, _vp]),
    "sparge_quantize_qk": (_i32, [_T, _T, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "sparge_hilbert_perm3d": (_i32, [_i32, _i32, _i32, _vp]),
    "sparge_reorder": (_i32, [_T, _T, _vp, _i64, _i64, _i32, _vp]),
    "sparge_status_str": (ctypes.c_char_p, [_i32]),
    "sparge_abi_version": (_i32, []),
}

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                path = lib_path()
                if not os.path.exists(path):
                    raise RuntimeError(
                        f"{path} is missing: build it with `python -m block_sparse_quantized_amd.build`"
                        " (there is no fallback implementation)")
                L = ctypes.CDLL(path)
                for name, (res, args) in PROTOTYPES.items():
                    fn = getattr(L, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = L
    return _lib
