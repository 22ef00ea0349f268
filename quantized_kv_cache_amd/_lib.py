"""ctypes declarations of libqkv.so's C ABI (include/qkv.h, include/qkv_measure.h)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqkv.so")

QKV_OK, QKV_EINVAL, QKV_EUNSUPPORTED, QKV_EWORKSPACE, QKV_EHIP = range(5)
STATUS_NAMES = {0: "QKV_OK", 1: "QKV_EINVAL", 2: "QKV_EUNSUPPORTED", 3: "QKV_EWORKSPACE",
                4: "QKV_EHIP"}
QKV_F32, QKV_F16, QKV_BF16 = 0, 1, 2
QKV_AFFINE, QKV_Q8_0, QKV_DENSE, QKV_QSYM = 0, 1, 2, 3
QKV_MASK_NONE, QKV_MASK_CAUSAL, QKV_MASK_ADDITIVE = 0, 1, 2
QKV_ALGO_AUTO, QKV_ALGO_GENERIC, QKV_ALGO_MATRIX, QKV_ALGO_UNFUSED, QKV_ALGO_DEQUANT_F16 = 0, 1, 2, 3, 4
QKV_KERNEL_GENERIC, QKV_KERNEL_DECODE, QKV_KERNEL_DECODE_NARROW, QKV_KERNEL_PREFILL = 0, 1, 2, 3
QKV_KERNEL_UNFUSED = 4
QKV_KERNEL_DECODE_STREAM = 5

# every symbol include/qkv.h declares
EXPORTS = ["qkv_quantize", "qkv_update_append", "qkv_dequantize", "qsdpa_workspace_bytes", "qsdpa_workspace_reset",
           "qsdpa_plan", "qsdpa_decode", "qsdpa_decode_static", "qsdpa_decode_append", "qsdpa_prefill",
           "qkv_last_error",
           "qkv_abi_version", "qkv_measure_read", "qkv_measure_read_config"]
QKV_TICKET_BYTES = 262144
QKV_STATIC_SCRATCH_BYTES = QKV_TICKET_BYTES + 16 * 1024 * 1024


class QkvPack(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("scale_dtype", ctypes.c_int32),
                ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("L_cap", ctypes.c_int64),
                ("D", ctypes.c_int64),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("biases", ctypes.c_void_p),
                ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_l", ctypes.c_int64)]


class QkvAttnOpts(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("algo", ctypes.c_int32),
                ("timing_events", ctypes.c_void_p * 2)]


class QkvAttnPlan(ctypes.Structure):
    _fields_ = [("algo", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("row_tile", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("keys_per_split", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t)]


class QKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load():
    """Load the in-tree libqkv.so; fails loudly when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m quantized_kv_cache_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    PK = ctypes.POINTER(QkvPack)
    OP = ctypes.POINTER(QkvAttnOpts)
    I64P = ctypes.POINTER(ctypes.c_int64)
    L.qkv_quantize.argtypes = [P, I32, I64P, I64, PK, P]
    L.qkv_quantize.restype = I32
    L.qkv_update_append.argtypes = [P, P, I32, I64P, I64, I64, PK, PK, P]
    L.qkv_update_append.restype = I32
    L.qkv_dequantize.argtypes = [PK, I64, PK, P]
    L.qkv_dequantize.restype = I32
    L.qsdpa_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, PK, I32, OP]
    L.qsdpa_workspace_bytes.restype = SZ
    L.qsdpa_workspace_reset.argtypes = [P, SZ, P]
    L.qsdpa_workspace_reset.restype = I32
    L.qsdpa_plan.argtypes = [I64, I64, I64, I64, I64, PK, I32, OP, ctypes.POINTER(QkvAttnPlan)]
    L.qsdpa_plan.restype = I32
    L.qsdpa_decode.argtypes = [P, I32, I64, I64, I64, PK, PK, I64, ctypes.c_float, P, I32, I64P,
                               P, P, SZ, OP, P]
    L.qsdpa_decode.restype = I32
    L.qsdpa_decode_static.argtypes = [P, I32, I64, I64, I64, PK, PK, I64, ctypes.c_float, P, I32,
                                      I64P, P, OP, P]
    L.qsdpa_decode_static.restype = I32
    L.qsdpa_decode_append.argtypes = [P, I32, I64, I64, I64, P, P, I64P, I64, PK, PK, ctypes.c_float, P, I32,
                                      I64P, P, P, SZ, OP, P]
    L.qsdpa_decode_append.restype = I32
    L.qsdpa_prefill.argtypes = [P, I32, I64, I64, I64, I64, PK, PK, I64, ctypes.c_float, I32, P,
                                I32, I64P, P, P, SZ, OP, P]
    L.qsdpa_prefill.restype = I32
    L.qkv_last_error.argtypes = []
    L.qkv_last_error.restype = ctypes.c_char_p
    L.qkv_abi_version.argtypes = []
    L.qkv_abi_version.restype = I32
    L.qkv_measure_read.argtypes = [P, SZ, I32, P, P]      # include/qkv_measure.h
    L.qkv_measure_read.restype = I32
    L.qkv_measure_read_config.argtypes = [P, SZ, I32, I32, I32, I32, P, P]
    L.qkv_measure_read_config.restype = I32
    _lib = L
    return L


def check(status: int) -> None:
    if status != QKV_OK:
        raise QKVError(status, load().qkv_last_error().decode())


def i64_array(vals):
    arr = (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])
    return arr
