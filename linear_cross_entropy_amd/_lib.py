"""ctypes view of libcce.so: the C ABI declared in include/cce.h."""
from __future__ import annotations

import ctypes
import os
import threading

from .build import LIB

STATUS = {
    0: "CCE_OK", 1: "CCE_ERR_NULL_POINTER", 2: "CCE_ERR_BAD_SHAPE",
    3: "CCE_ERR_BAD_REDUCTION", 4: "CCE_ERR_BAD_ALIGNMENT", 5: "CCE_ERR_BAD_EPS",
    6: "CCE_ERR_WORKSPACE_TOO_SMALL", 7: "CCE_ERR_HIP", 8: "CCE_ERR_BAD_FILTER_MODE",
    9: "CCE_ERR_SCRATCH_TOO_SMALL",
}

EXPORTS = (
    "cce_workspace_bytes", "cce_forward", "cce_backward", "cce_backward_ex", "cce_vocab_order",
    "cce_backward_sorted", "cce_status_string", "cce_profile_enable", "cce_profile_query",
    "cce_forward_noalloc",
)


class CCEError(RuntimeError):
    def __init__(self, code: int, what: str, msg: str):
        super().__init__(f"{what}: {STATUS.get(code, code)} ({msg})")
        self.code = code


class FilterStats(ctypes.Structure):
    _fields_ = [("units_total", ctypes.c_int64), ("units_skipped", ctypes.c_int64),
                ("unit_rows", ctypes.c_int32), ("unit_cols", ctypes.c_int32)]


_lock = threading.Lock()
_lib = None


def load():
    """Load the in-tree library; raises if it has not been built (there is no fallback)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB):
            raise ImportError(
                f"{LIB} is missing: build it with linear_cross_entropy_amd.build.build() "
                "(or __graft_entry__.build()); there is no CPU fallback")
        lib = ctypes.CDLL(LIB)
        i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        lib.cce_workspace_bytes.argtypes = [i64, i64, i64, ctypes.POINTER(sz), ctypes.POINTER(sz)]
        lib.cce_forward.argtypes = [vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, sz, vp]
        lib.cce_forward_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, vp, vp,
                                            vp]
        lib.cce_backward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                     ctypes.c_float, vp, vp, vp, vp, sz, vp]
        lib.cce_backward_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                        ctypes.c_float, ctypes.c_int, vp, vp, vp, vp, sz, vp]
        lib.cce_vocab_order.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, vp, sz, vp]
        lib.cce_backward_sorted.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                            ctypes.c_float, ctypes.c_int, vp, vp, vp, vp, vp, sz,
                                            vp]
        lib.cce_status_string.argtypes = [ctypes.c_int]
        lib.cce_status_string.restype = ctypes.c_char_p
        lib.cce_profile_enable.argtypes = [ctypes.c_int]
        lib.cce_profile_query.argtypes = [ctypes.c_char_p, ctypes.POINTER(i64),
                                          ctypes.POINTER(ctypes.c_double)]
        for name in EXPORTS:
            if name != "cce_status_string":
                getattr(lib, name).restype = ctypes.c_int
        _lib = lib
        return lib


def check(code: int, what: str):
    if code != 0:
        msg = load().cce_status_string(code).decode()
        raise CCEError(code, what, msg)
