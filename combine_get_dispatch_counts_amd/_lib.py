"""ctypes declarations for libepx.so (the C ABI in include/epx.h).

Loading fails loudly: there is no fallback path. Build the library with
``python -m combine_get_dispatch_counts_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libepx.so")

EPX_OK, EPX_EINVAL, EPX_ECAPACITY, EPX_EUNSUPPORTED, EPX_EHIP, EPX_EDEVICE = 0, -1, -2, -3, -4, -5
DEV_BAD_ROUTE, DEV_OVERFLOW, DEV_BAD_HANDLE, DEV_WORKSPACE = 1, 2, 4, 8
MAX_TOPK, MAX_EXPERTS, MAX_RANKS, MAX_SWEEP_GBPS = 32, 512, 64, 100000
NOALLOC_SCRATCH_BYTES = 1 << 20

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); the order follows include/epx.h
SIGNATURES = {
    "epx_create": (_I, [ctypes.POINTER(_P), _I]),
    "epx_destroy": (_I, [_P]),
    "epx_strerror": (ctypes.c_char_p, [_I]),
    "epx_set_sweep_rate": (_I, [_P, _I, _I]),
    "epx_get_sweep_rate": (_I, [_P, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "epx_calibrate_sweep_rate": (_I, [_P, _P, _SZ, ctypes.POINTER(_I), _P]),
    "epx_workspace_size": (_I, [_I, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "epx_ll_size_hint": (_SZ, [_I, _I, _I, _I, _I]),
    "epx_scale_stride": (_I, [_I]),
    "epx_get_dispatch_layout": (_I, [_P, _P, _I, _I, _I, _I, _I] + [_P] * 11 + [_SZ, _P]),
    "epx_get_dispatch_layout_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _I] + [_P] * 10 + [_P]),
    "epx_dispatch": (_I, [_P, _P, _I, _P, _P, _I, _I, _I, _I] + [_P] * 4 + [_I]
                     + [_P] * 5 + [_I64] + [_P] * 3 + [_I64, _P, _P]),
    "epx_permute": (_I, [_P, _P, _I, _P, _I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _I64, _P, _P]),
    "epx_fused_workspace_size": (_I, [_I, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "epx_fused_launches": (_I, [_P] + [_I] * 6 + [ctypes.POINTER(_I)]),
    "epx_dispatch_fused": (_I, [_P, _P, _I, _P, _P, _I, _I, _I, _I, _I] + [_P] * 11 + [_SZ, _I]
                           + [_P] * 5 + [_I64] + [_P] * 3 + [_I64, _P, _P]),
    "epx_combine": (_I, [_P, _P, _I64, _I, _P, _P, _I, _I, _P, _P]),
    "epx_combine_partial": (_I, [_P, _P, _I64, _I, _P, _P, _P, _P, _I, _I, _I64, _P, _P, _P]),
    "epx_combine_final": (_I, [_P, _P, _I64, _I, _P, _P, _I, _I, _P, _P]),
    "epx_ll_reset": (_I, [_P, _P, _I64, _P]),
    "epx_ll_dispatch": (_I, [_P, _P, _I, _P] + [_I] * 8 + [_P] * 5 + [_P, _I64, _P, _P]),
    "epx_get_error": (_I, [_P, ctypes.POINTER(_I), _P]),
}

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m combine_get_dispatch_counts_amd.build` (there is no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class EpxError(RuntimeError):
    def __init__(self, code: int, what: str, flags: int = 0):
        msg = load().epx_strerror(code).decode()
        extra = f" (device flags {flags:#x})" if flags else ""
        super().__init__(f"{what}: {msg} [{code}]{extra}")
        self.code = code
        self.flags = flags


def check(rc: int, what: str) -> None:
    if rc != EPX_OK:
        raise EpxError(rc, what)
