"""ctypes declarations of the C ABI in include/awq.h (libawq_gfx950.so).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libawq_gfx950.so")

AWQ_OK = 0
STATUS_NAMES = {0: "AWQ_OK", 1: "AWQ_ERR_NULL", 2: "AWQ_ERR_SHAPE", 3: "AWQ_ERR_DTYPE",
                4: "AWQ_ERR_ALIGN", 5: "AWQ_ERR_UNSUPPORTED", 6: "AWQ_ERR_WORKSPACE",
                7: "AWQ_ERR_HIP"}
AWQ_F16, AWQ_BF16, AWQ_F32 = 0, 1, 2
AWQ_OP_ACT_STATS, AWQ_OP_SEARCH, AWQ_OP_QUANTIZE, AWQ_OP_GEMM = 0, 1, 2, 3
AWQ_GROUP = 128
AWQ_MAX_ALPHA = 64
AWQ_NOALLOC_SCRATCH_BYTES = 128 << 20

# exported symbol -> (restype, argtypes)
_i64, _p, _i, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "awq_abi_version": (ctypes.c_int, []),
    "awq_status_str": (ctypes.c_char_p, [_i]),
    "awq_workspace_bytes": (_sz, [_i, _i64, _i64, _i64, _i64, _i]),
    "awq_act_stats": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _sz, _p]),
    "awq_search_scales": (_i, [_p, _i, _i64, _i64, _p, _i64, _i64, _p, _p, _i, _i, _p, _p, _p, _p,
                               _p, _sz, _p]),
    "awq_search_scales_ex": (_i, [_p, _i, _i64, _i64, _p, _i64, _i64, _p, _p, _i, _i, _i, _i, _p, _p,
                                  _p, _p, _p, _p, _sz, _p]),
    "awq_salient_channels": (_i, [_p, _i64, _i64, _p, _p]),
    "awq_quantize_pack": (_i, [_p, _i, _i64, _i64, _p, _i, _p, _p, _p, _p, _p]),
    "awq_quantize_codes": (_i, [_p, _i, _i64, _i64, _p, _i, _i, _i, _p, _p, _p, _p]),
    "awq_w4a16_gemm": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _p, _i64, _i, _p, _p, _i, _i64, _p,
                            _sz, _p]),
    "awq_fold_scales": (_i, [_p, _i, _i64, _i64, _i64, _p, _i, _p]),
    "awq_w4a16_gemm_noalloc": (_i, [_p, _i, _i64, _i64, _i64, _p, _p, _p, _i64, _i, _p, _p, _i, _i64,
                                    _p]),
    "awq_read_stream": (_i, [_p, _i64, _i, _i, _p, _p]),
}

_lib = None


class AwqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} "
                         f"({lib().awq_status_str(status).decode()})")


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the gfx950 HIP library first "
                "(python -m weight_only_int4_stats_amd.build); there is no fallback path")
        handle = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(fn: str, status: int) -> None:
    if status != AWQ_OK:
        raise AwqError(fn, status)
