"""ctypes declarations of libfp4bs.so, mirroring include/fp4bs.h one to one."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp4bs.so")

FP4_OK, FP4_EINVAL, FP4_EUNSUPPORTED, FP4_EALIGN, FP4_EHIP, FP4_ERANGE = range(6)
STATUS_NAMES = {0: "FP4_OK", 1: "FP4_EINVAL", 2: "FP4_EUNSUPPORTED", 3: "FP4_EALIGN", 4: "FP4_EHIP", 5: "FP4_ERANGE"}
FP4_UE5M3, FP4_E4M3, FP4_E8M0 = 0, 1, 2
FP4_VIEW_ROW, FP4_VIEW_COL, FP4_VIEW_TILE2D = 0, 1, 2
FP4_IN_BF16, FP4_IN_FP32 = 0, 1
FP4_SCALES_1D, FP4_SCALES_2D, FP4_SCALES_2D_T = 0, 1, 2
ABI_VERSION = 3

EXPORTED = [
    "fp4_quantize", "fp4_quantize_rowcol", "fp4_fake_quant", "fp4_dequantize", "fp4_mxfp4_to_fp8", "fp4_quantize_local", "fp4_quantize_sizes", "fp4_tensor_amax", "amax_cache_update", "amax_cache_reset",
    "fp4_gemm_fprop", "fp4_gemm_dgrad", "fp4_gemm_wgrad", "fp4_gemm_fprop_q", "fp4_gemm_dgrad_q",
    "fp4_scale_range", "fp4_gemm_check_range", "fp4_decode_f16", "fp4_gemm_f16",
    "fp4_debug_encode", "fp4_last_error", "fp4_abi_version",
]


class QuantCfg(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("block", ctypes.c_int32), ("view", ctypes.c_int32),
                ("stochastic", ctypes.c_int32), ("hadamard_n", ctypes.c_int32), ("T", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64)]


class Operand(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p), ("g", ctypes.c_void_p),
                ("fmt", ctypes.c_int32), ("block", ctypes.c_int32), ("scale_layout", ctypes.c_int32),
                ("g_stripe", ctypes.c_int32), ("rows", ctypes.c_int64), ("k", ctypes.c_int64)]


class AmaxCacheC(ctypes.Structure):
    _fields_ = [("amax", ctypes.c_void_p), ("valid", ctypes.c_void_p), ("D", ctypes.c_int32)]


_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

SIGNATURES = {
    "fp4_quantize": ([_P, _I32, _I64, _I64, _I64, ctypes.POINTER(QuantCfg), _P, _P, _P, _P, _P, _P, _P, _P],
                     ctypes.c_int),
    "fp4_quantize_rowcol": ([_P, _I32, _I64, _I64, _I64, ctypes.POINTER(QuantCfg), ctypes.POINTER(QuantCfg), _P, _P,
                             _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "fp4_fake_quant": ([_P, _I32, _I64, _I64, _I64, ctypes.POINTER(QuantCfg), _P, _P, _I32, _I64, _P], ctypes.c_int),
    "fp4_dequantize": ([ctypes.POINTER(Operand), _P, _I32, _I64, _P], ctypes.c_int),
    "fp4_mxfp4_to_fp8": ([ctypes.POINTER(Operand), _I32, _P, _P, _P], ctypes.c_int),
    "fp4_quantize_local": ([_P, _I32, _I64, _I64, _I64, ctypes.POINTER(QuantCfg), _I32, _P, _P, _P, _P, _P],
                           ctypes.c_int),
    "fp4_quantize_sizes": ([_I64, _I64, ctypes.POINTER(QuantCfg), ctypes.POINTER(_SZ), ctypes.POINTER(_SZ),
                            ctypes.POINTER(_SZ)], ctypes.c_int),
    "fp4_tensor_amax": ([_P, _I32, _I64, _I64, _I64, _I32, _P, _P], ctypes.c_int),
    "amax_cache_update": ([ctypes.POINTER(AmaxCacheC), _I64, _P, _P], ctypes.c_int),
    "amax_cache_reset": ([ctypes.POINTER(AmaxCacheC), _P], ctypes.c_int),
    "fp4_gemm_fprop": ([ctypes.POINTER(Operand), ctypes.POINTER(Operand), _P, _I32, _P], ctypes.c_int),
    "fp4_gemm_dgrad": ([ctypes.POINTER(Operand), ctypes.POINTER(Operand), _P, _I32, _P], ctypes.c_int),
    "fp4_gemm_wgrad": ([ctypes.POINTER(Operand), ctypes.POINTER(Operand), _P, _I32, _I32, _P], ctypes.c_int),
    "fp4_gemm_fprop_q": ([ctypes.POINTER(Operand), ctypes.POINTER(Operand), _P, _I32, ctypes.POINTER(QuantCfg), _P,
                          _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "fp4_gemm_dgrad_q": ([ctypes.POINTER(Operand), ctypes.POINTER(Operand), _P, _I32, ctypes.POINTER(QuantCfg), _P,
                          _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "fp4_scale_range": ([ctypes.POINTER(Operand), _P, _P], ctypes.c_int),
    "fp4_gemm_check_range": ([_I32, ctypes.POINTER(_I32), ctypes.POINTER(_I32)], ctypes.c_int),
    "fp4_decode_f16": ([ctypes.POINTER(Operand), _P, _P], ctypes.c_int),
    "fp4_gemm_f16": ([ctypes.POINTER(Operand), _P, ctypes.POINTER(Operand), _P, _P, _I32, _I32, _P], ctypes.c_int),
    "fp4_debug_encode": ([_P, _P, _I64, _I32, _P, _P], ctypes.c_int),
    "fp4_last_error": ([], ctypes.c_char_p),
    "fp4_abi_version": ([], ctypes.c_int32),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m fp4_block_scaled_tensor_amd.build` "
                          "(the FP4 path has no CPU or PyTorch fallback)")
    lib = ctypes.CDLL(path)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if lib.fp4_abi_version() != ABI_VERSION:
        raise ImportError(f"libfp4bs ABI {lib.fp4_abi_version()} != expected {ABI_VERSION}")
    _lib = lib
    return lib


class FP4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def check(status: int) -> None:
    if status != FP4_OK:
        raise FP4Error(status, load().fp4_last_error().decode())
