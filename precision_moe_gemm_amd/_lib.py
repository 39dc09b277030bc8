"""ctypes loader for libnvfp4.so (argument marshalling only).

The library is built in-tree by ``precision_moe_gemm_amd.build``.  Loading
fails loudly when it is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
# NVFP4_LIB_PATH selects another build of the same sources (the sanitizer
# build of the host layer); it must carry the same source stamp
LIB_PATH = os.environ.get("NVFP4_LIB_PATH") or os.path.join(HERE, "libnvfp4.so")

_lock = threading.Lock()
_lib = None

OK, INVALID_ARG, SHAPE, RANGE, WORKSPACE, DEVICE, UNSUPPORTED, DATA = range(8)
F32, BF16 = 0, 1
OP_QUANTIZE, OP_REMAP, OP_GEMM, OP_MOE, OP_MOE_ROUTE, OP_MX_MOE = range(6)


class NVFP4TensorC(ctypes.Structure):
    _fields_ = [
        ("packed", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("global_", ctypes.c_void_p),
        ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64),
        ("batch", ctypes.c_int64),
        ("flags", ctypes.c_uint32),
    ]


POW2_SCALES = 1  # NVFP4_POW2_SCALES
TILED_SCALES = 2  # NVFP4_TILED_SCALES


# name -> (restype, argtypes); mirrors include/nvfp4.h
P = ctypes.c_void_p
I64 = ctypes.c_int64
I32 = ctypes.c_int32
SZ = ctypes.c_size_t
ST = ctypes.c_int
TP = ctypes.POINTER(NVFP4TensorC)
SIGNATURES = {
    "nvfp4_workspace_size": (SZ, [ctypes.c_int, I64, I32, I32, I64, I64]),
    "nvfp4_quantize": (ST, [P, I64, I64, I64, P, TP, P, SZ, P]),
    "nvfp4_dequantize": (ST, [TP, P, ctypes.c_int, P]),
    "nvfp4_gather_dequantize": (ST, [TP, P, I64, P, I32, P]),
    "nvfp4_tile_scales": (ST, [TP, P, P]),
    "mxfp4_quantize": (ST, [P, I64, I64, I64, P, P, P]),
    "mxfp4_to_nvfp4": (ST, [P, P, I64, I64, I64, TP, P, SZ, P]),
    "nvfp4_gemm": (ST, [TP, TP, P, ctypes.c_int, P, SZ, P]),
    "nvfp4_moe_grouped_gemm": (ST, [P, P, P, I64, I32, I32, TP, TP, P, P, P, SZ, P]),
    "nvfp4_gemm_w4a16": (ST, [P, I64, I64, I64, TP, P, ctypes.c_int, P, SZ, P]),
    "mxfp8_quantize": (ST, [P, I64, I64, I64, P, P, P]),
    "mx_gemm_w4a8": (ST, [P, P, I64, I64, P, P, I64, P, ctypes.c_int, P]),
    "mx_moe_w4a8": (ST, [P, P, P, I64, ctypes.c_int32, ctypes.c_int32, I64, I64, P, P, P, P, P, P, ctypes.c_size_t, P]),
    "mx_moe_gate_up": (ST, [P, P, P, P, I64, ctypes.c_int32, ctypes.c_int32, I64, I64, P, P, P, P, P, ctypes.c_size_t,
                            P]),
    "mx_moe_down": (ST, [P, P, P, I64, ctypes.c_int32, ctypes.c_int32, I64, I64, P, P, P, P, ctypes.c_size_t, P]),
    "nvfp4_moe_w4a16": (ST, [P, P, P, I64, I32, I32, TP, TP, P, P, SZ, P]),
    "nvfp4_moe_grouped_gemm_noalloc": (ST, [P, P, P, I64, I32, I32, TP, TP, P, P, P]),
    "nvfp4_noalloc_scratch_bytes": (SZ, []),
    "nvfp4_moe_route": (ST, [P, I64, I32, I32, P, P, P, P, SZ, P]),
    "nvfp4_moe_gate_up": (ST, [TP, P, P, I64, I32, I32, TP, P, P, P, SZ, P]),
    "nvfp4_moe_gate_up_q": (ST, [TP, P, P, I64, I32, I32, TP, P, TP, P, SZ, P]),
    "nvfp4_moe_down": (ST, [TP, P, I64, I32, I32, TP, P, P, SZ, P]),
    "nvfp4_moe_combine": (ST, [P, P, P, I64, I32, I64, P, P]),
    "nvfp4_kv_quant": (ST, [P, P, I64, I64, I64, TP, TP, P]),
    "nvfp4_kv_dequant": (ST, [TP, TP, I64, I64, I64, P, P, ctypes.c_int, P]),
    "nvfp4_audit_scales": (ST, [TP, P, P]),
    "nvfp4_get_error": (ST, [P]),
    "nvfp4_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "nvfp4_recipe": (None, [ctypes.POINTER(ctypes.c_int32)]),
    "nvfp4_build_stamp": (ctypes.c_char_p, []),
    "nvfp4_set_checks": (ctypes.c_int, [ctypes.c_int]),
}


def load():
    """Load libnvfp4.so; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libnvfp4.so not found at {LIB_PATH}; build it with "
                "`python -m precision_moe_gemm_amd.build` (there is no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        from .build import source_hash
        lib.nvfp4_build_stamp.restype = ctypes.c_char_p
        lib.nvfp4_build_stamp.argtypes = []
        stamp, want = lib.nvfp4_build_stamp().decode(), source_hash()
        if stamp != want:
            raise ImportError(
                f"libnvfp4.so at {LIB_PATH} was built from other sources (stamp {stamp}, sources {want}); "
                "rebuild it with `python -m precision_moe_gemm_amd.build`")
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib
