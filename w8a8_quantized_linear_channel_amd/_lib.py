"""ctypes loader for libq8.so (the C ABI declared in include/q8.h, and the
measurement helper of include/q8_bench.h).

Argument marshalling only: this module never computes anything itself.  If
the library has not been built the loader raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libq8.so")

# enum values, as in include/q8.h
Q8_OK = 0
STATUS_NAMES = {
    0: "Q8_OK", 1: "Q8_ERR_NULL_PTR", 2: "Q8_ERR_BAD_SHAPE", 3: "Q8_ERR_BAD_DTYPE",
    4: "Q8_ERR_BAD_FORMAT", 5: "Q8_ERR_BAD_ARG", 6: "Q8_ERR_ALIGN", 7: "Q8_ERR_WORKSPACE",
    8: "Q8_ERR_DEVICE", 9: "Q8_ERR_LAUNCH",
}
Q8_F32, Q8_F16, Q8_BF16 = 0, 1, 2
Q8_INT8_ASYM, Q8_INT8_SYM, Q8_FP8_E4M3 = 0, 1, 2
Q8_OP_LINEAR, Q8_OP_DECOMP, Q8_OP_FP8, Q8_OP_STATIC, Q8_OP_GROUPED = 0, 1, 2, 3, 4

# every symbol include/q8.h declares, with (restype, argtypes)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
SIGNATURES = {
    "q8_quantize_weight": (_INT, [_INT, _P, _INT, _I64, _I64, _P, _P, _P, _P]),
    "q8_quantize_act": (_INT, [_INT, _P, _INT, _I64, _I64, _F, _P, _P, _P, _P]),
    "q8_linear": (_INT, [_P, _INT, _I64, _I64, _P, _P, _P, _I64, _P, _P, _INT, _P, _SZ, _P, _P]),
    "q8_linear_int8_decomp": (_INT, [_P, _I64, _I64, _P, _P, _P, _I64, _F, _P, _P, _P, _SZ, _P, _P,
                                     _P, _P]),
    "q8_linear_fp8": (_INT, [_P, _I64, _I64, _P, _P, _I64, _F, _P, _P, _P, _SZ, _P]),
    "q8_gemm_int8": (_INT, [_P, _P, _P, _I64, _I64, _P, _P, _P, _I64, _P, _P, _INT, _P, _P]),
    "q8_gemm_fp8": (_INT, [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P, _P]),
    "q8_linear_w8a16": (_INT, [_P, _INT, _I64, _I64, _P, _P, _P, _I64, _P, _P, _INT, _P]),
    "q8_linear_fp8_grouped": (_INT, [_P, _I64, _I64, _P, _I64, _P, _P, _I64, _F, _P, _P, _SZ, _P]),
    "q8_quantize_act_static": (_INT, [_P, _INT, _I64, _I64, _F, _P, _P, _P]),
    "q8_linear_static": (_INT, [_P, _INT, _I64, _I64, _F, _P, _P, _P, _I64, _P, _F, _P, _P, _SZ, _P]),
    "q8_quantize_weight_grouped": (_INT, [_P, _INT, _I64, _I64, _I64, _P, _P, _P, _P]),
    "q8_linear_grouped": (_INT, [_P, _INT, _I64, _I64, _P, _P, _P, _I64, _I64, _P, _P, _INT, _P, _SZ, _P]),
    "q8_linear_noalloc": (_INT, [_P, _INT, _I64, _I64, _P, _P, _P, _I64, _P, _P, _INT, _P, _P]),
    "q8_workspace_bytes": (_SZ, [_INT, _I64, _I64, _I64]),
    # include/q8_bench.h
    "q8_bench_mfma_loop": (_INT, [_INT, _I64, _I64, _P, _P]),
    "q8_probe_fp8_mfma": (_INT, [_P, _P, _P, _P, _I64, _P]),
    "q8_bench_stream_read": (_INT, [_P, _I64, _I64, _P, _P]),
    "q8_gemm_tile": (_INT, [_INT, _I64, _I64, _I64, _P, _P]),
    "q8_status_str": (ctypes.c_char_p, [_INT]),
}

_LIB = None


class Q8Error(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} returned {STATUS_NAMES.get(status, status)}")


def lib() -> ctypes.CDLL:
    """Load libq8.so once; raise if it is missing (build it first)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libq8.so is not built ({LIB_PATH}); run `python -c \"import __graft_entry__ as g; "
                f"g.build()\"` or `python w8a8_quantized_linear_channel_amd/build.py`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _LIB = h
    return _LIB


def check(func: str, status: int) -> None:
    if status != Q8_OK:
        raise Q8Error(func, status)
