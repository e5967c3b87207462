"""ctypes view of libfa.so's C ABI (include/fa.h). Argument marshalling only."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_FP32, FA_FP16, FA_BF16 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)

# Every symbol include/fa.h declares, with (restype, argtypes).
_P, _I64, _F, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
_U64 = ctypes.c_uint64
PROTOTYPES = {
    "fa_forward": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _F, _I, _I, _P]),
    "fa_forward_varlen": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                         _I64, _F, _I, _I, _P]),
    "fa_forward_dropout": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _F, _I, _I,
                                          _F, _U64, _U64, _P]),
    "fa_backward_dropout": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I64,
                                           _I64, _I64, _I64, _F, _I, _I, _F, _U64, _U64, _P]),
    "fa_backward_varlen": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I64,
                                          _I64, _I64, _I64, _I64, _I64, _F, _I, _I, _P]),
    "fa_backward_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64]),
    "fa_decode_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I64, _I64]),
    "fa_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _SZ, _I64, _I64, _I64, _I64, _I64,
                                 _I64, _I64, _F, _I, _P]),
    "fa_backward": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I64, _I64,
                                   _I64, _I64, _F, _I, _I, _P]),
    "fa_backward_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64,
                                           _I64, _F, _I, _I, _P]),
    "fa_forward_gqa": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _I,
                                      _I, _F, _U64, _U64, _P]),
    "fa_backward_gqa": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I64, _I64,
                                       _I64, _I64, _I64, _F, _I, _I, _F, _U64, _U64, _P]),
    "fa_forward_varlen_dropout": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64,
                                                 _I64, _I64, _F, _I, _I, _F, _U64, _U64, _P]),
    "fa_backward_varlen_dropout": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                                  _I64, _I64, _I64, _I64, _I64, _I64, _F, _I, _I,
                                                  _F, _U64, _U64, _P]),
    "fa_clock_probe": (ctypes.c_int, [_P, _I, _P]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_last_error": (ctypes.c_char_p, []),
}

_lib = None


class FaError(RuntimeError):
    """A libfa call returned a non-zero fa_status."""

    def __init__(self, fn, status, detail):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)}: {detail}")


def load():
    """Load libfa.so once; fail loudly if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (exact_attention_113_amd.build.build())")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status):
    return load().fa_status_string(int(status)).decode()


def last_error():
    return load().fa_last_error().decode()


def check(fn, status):
    if status != FA_OK:
        raise FaError(fn, status, last_error())
