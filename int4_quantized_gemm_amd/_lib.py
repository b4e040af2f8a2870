"""ctypes declarations of libtp.so (the C ABI in include/tp.h).

The library is loaded on first use. There is no fallback: if libtp.so has not
been built, every call raises.
"""

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtp.so")

TP_OK = 0
STATUS_NAMES = {
    0: "TP_OK",
    1: "TP_ERR_NULL_POINTER",
    2: "TP_ERR_BAD_SHAPE",
    3: "TP_ERR_K_NOT_MULTIPLE_OF_256",
    4: "TP_ERR_BAD_LEADING_DIM",
    5: "TP_ERR_MISALIGNED",
    6: "TP_ERR_UNSUPPORTED_DTYPE",
    7: "TP_ERR_UNSUPPORTED_BITS",
    8: "TP_ERR_SIZE_OVERFLOW",
    9: "TP_ERR_WORKSPACE_TOO_SMALL",
    10: "TP_ERR_BAD_ALIASING",
    11: "TP_ERR_BAD_FLAGS",
    12: "TP_ERR_HIP",
}
TP_F32, TP_BF16 = 0, 1
TP_A_PREROTATED, TP_A_ROTATE = 0, 1
TP_OP_QGEMM_W8, TP_OP_QGEMM_W4, TP_OP_QGEMM_W8A8, TP_OP_QGEMM_W8A8_PREQUANTIZED = 1, 2, 3, 4
TP_OP_QGEMM_W4A8, TP_OP_QGEMM_W4A8_PREQUANTIZED = 5, 6
TP_FFN_OUT_I8, TP_FFN_OUT_BF16 = 0, 1

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "tp_rotate_quantize_weights": (_int, [_p, _int, _i64, _i64, _i64, _int, _p, _i64, _p, _p]),
    "tp_hadamard_rotate_rows": (_int, [_p, _int, _i64, _i64, _i64, _p, _int, _i64, _p]),
    "tp_quantize_rows_int8": (_int, [_p, _int, _i64, _i64, _i64, _int, _p, _i64, _p, _p]),
    "tp_lora_workspace_size": (_sz, [_i64, _i64]),
    "tp_lora_add": (_int, [_p, _int, _i64, _p, _p, _int, _i64, _i64, ctypes.c_float, _i64, _i64, _i64, _i64, _p, _int,
                           _i64, _p, _sz, _p]),
    "tp_lora_down": (_int, [_p, _int, _i64, _p, _int, _i64, _i64, _i64, _i64, _p, _sz, _p]),
    "tp_qgemm_w8a8_prequantized_lora": (_int, [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _i64, _p, _i64, _p, _p, _i64,
                                               _i64, ctypes.c_float, _p, _sz, _p]),
    "tp_dequantize_unrotate": (_int, [_p, _int, _i64, _p, _i64, _i64, _p, _int, _i64, _p]),
    "tp_requantize_weights": (_int, [_p, _int, _i64, _p, _i64, _i64, _int, _p, _i64, _p, _p]),
    "tp_swiglu_rotate": (_int, [_p, _i64, _p, _i64, _int, _i64, _i64, _int, _p, _i64, _p, _p]),
    "tp_workspace_size": (_sz, [_int, _i64, _i64, _i64, _int]),
    "tp_qgemm_w8": (_int, [_p, _int, _i64, _int, _p, _i64, _p, _i64, _i64, _i64, _p, _int, _i64, _p, _sz, _p]),
    "tp_qgemm_w4": (_int, [_p, _int, _i64, _int, _p, _i64, _p, _i64, _i64, _i64, _p, _int, _i64, _p, _sz, _p]),
    "tp_qgemm_w8a8": (_int, [_p, _int, _i64, _int, _p, _i64, _p, _i64, _i64, _i64, _p, _int, _i64,
                              _p, _p, _p, _i64, _p, _sz, _p]),
    "tp_qgemm_w8a8_prequantized": (_int, [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _i64, _p, _int, _i64, _p, _i64,
                                           _p, _sz, _p]),
    "tp_qgemm_w8a8_prequantized_noalloc": (_int, [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _i64, _p, _int, _i64, _p,
                                                   _i64, _p]),
    "tp_qgemm_w4a8": (_int, [_p, _int, _i64, _int, _p, _i64, _p, _i64, _i64, _i64, _p, _int, _i64, _p, _p, _p,
                             _sz, _p]),
    "tp_qgemm_w4a8_prequantized": (_int, [_p, _i64, _p, _p, _i64, _p, _i64, _i64, _i64, _p, _int, _i64, _p, _sz,
                                          _p]),
    "tp_status_string": (ctypes.c_char_p, [_int]),
    "tp_last_error_message": (ctypes.c_char_p, []),
    "tp_abi_version": (_int, []),
}

_lock = threading.Lock()
_lib = None


class TPError(RuntimeError):
    """A libtp call returned a status other than TP_OK."""

    def __init__(self, status, message):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, f"status {status}")
        super().__init__(f"{self.status_name}: {message}")


def load():
    """Load libtp.so once and declare its symbols. Raises if it is missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                    "(there is no non-HIP fallback)")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
        return _lib


def check(status):
    if status != TP_OK:
        msg = load().tp_last_error_message().decode(errors="replace")
        raise TPError(status, msg)
