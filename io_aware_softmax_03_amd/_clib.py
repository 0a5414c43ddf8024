"""ctypes view of the C ABI in include/fa.h (no torch here).

Loading fails loudly when the shared library has not been built: there is no
CPU or PyTorch fallback for any entry point.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_HEADDIM = 0, -1, -2, -3
FA_ERR_DTYPE, FA_ERR_WORKSPACE, FA_ERR_ARG, FA_ERR_HIP, FA_ERR_SCRATCH = -4, -5, -6, -7, -8
FA_DTYPE_F32, FA_DTYPE_BF16 = 0, 1

# every symbol include/fa.h declares, with (restype, argtypes)
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "fa_strerror": (ctypes.c_char_p, [_I]),
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_fwd_window": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I, _P]),
    "fa_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_fwd_fp8_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "fa_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _Z, _P]),
    "fa_bwd_workspace_bytes": (_Z, [_I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P, _Z, _P]),
    "fa_decode_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "fa_decode": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P, _Z, _P]),
    "fa_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _Z, _P]),
}


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m io_aware_softmax_03_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def strerror(status: int) -> str:
    return lib().fa_strerror(status).decode()


def check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FAError(status, where)
