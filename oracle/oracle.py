"""ctypes front end of the C oracle (``qkv_oracle.c``).

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing).

Array conventions (numpy, C-contiguous):
  * ``"f32"`` values are ``np.float32``; ``"f16"`` values are ``np.float16``;
    ``"bf16"`` values are ``np.uint16`` bit patterns.
  * affine and symmetric 4/5-bit ("qsym") codes are ``np.uint32`` words
    holding each row's least-significant-bit-first code stream; Q8_0 codes are
    ``np.int8``; Q8_0 and qsym scales are fp16 bit patterns (``np.uint16``).

Every wrapper only marshals arrays; the arithmetic is in the C file, where
each function cites the page passage it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qkv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
_NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}

__all__ = [
    "build", "lib", "num_threads", "DTYPE_CODE",
    "f16_bits_from_f32", "f32_from_f16_bits", "bf16_bits_from_f32", "f32_from_bf16_bits",
    "to_f32", "affine_eps",
    "quantize_affine", "dequant_affine", "quantize_q8_0", "dequant_q8_0", "quantize_qsym",
    "dequant_qsym",
    "append_rows", "attention", "quantize", "dequant",
]


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (plain C, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.check_call(cmd)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_affine_eps.argtypes = [I]
        L.orc_affine_eps.restype = ctypes.c_float
        L.orc_quantize_affine.argtypes = [P, I, I64, I64, I, I, I, P, P, P]
        L.orc_quantize_affine.restype = None
        L.orc_dequant_affine.argtypes = [P, P, P, I, I64, I64, I, I, P]
        L.orc_dequant_affine.restype = None
        L.orc_quantize_q8_0.argtypes = [P, I, I64, I64, P, P]
        L.orc_quantize_q8_0.restype = None
        L.orc_dequant_q8_0.argtypes = [P, P, I64, I64, P]
        L.orc_dequant_q8_0.restype = None
        L.orc_quantize_qsym.argtypes = [P, I, I64, I64, I, P, P]
        L.orc_quantize_qsym.restype = None
        L.orc_dequant_qsym.argtypes = [P, P, I64, I64, I, P]
        L.orc_dequant_qsym.restype = None
        L.orc_attention.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, ctypes.c_double,
                                    P, P, I, P]
        L.orc_attention.restype = None
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = I
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().orc_num_threads())


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    a = np.asarray(a)
    if dtype is not None and a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


# --------------------------------------------------------------------------- scalar formats
def f16_bits_from_f32(x) -> np.ndarray:
    x = _c(np.asarray(x, dtype=np.float32))
    f = lib().orc_f32_to_f16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def f32_from_f16_bits(h) -> np.ndarray:
    h = _c(np.asarray(h, dtype=np.uint16))
    f = lib().orc_f16_to_f32
    return np.array([f(int(v)) for v in h.ravel()], dtype=np.float32).reshape(h.shape)


def bf16_bits_from_f32(x) -> np.ndarray:
    x = _c(np.asarray(x, dtype=np.float32))
    f = lib().orc_f32_to_bf16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def f32_from_bf16_bits(h) -> np.ndarray:
    h = _c(np.asarray(h, dtype=np.uint16))
    f = lib().orc_bf16_to_f32
    return np.array([f(int(v)) for v in h.ravel()], dtype=np.float32).reshape(h.shape)


def to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen a stored array to fp32 (exact for all three formats).  fp16 uses
    numpy's IEEE widening (a library primitive), bf16 the bit-pattern shift."""
    a = np.ascontiguousarray(a)
    if dtype == "f32":
        return a.astype(np.float32)
    if dtype == "f16":
        return a.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (a.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def affine_eps(scale_dtype: str) -> float:
    return float(lib().orc_affine_eps(DTYPE_CODE[scale_dtype]))


# --------------------------------------------------------------------------- quantizers
def quantize_affine(x: np.ndarray, dtype: str, bits: int, group_size: int,
                    scale_dtype: str | None = None):
    """Affine group quantize the last axis of ``x``.  Returns (codes, scales, biases)."""
    scale_dtype = scale_dtype or dtype
    x = _c(x, _NP_STORAGE[dtype])
    D = x.shape[-1]
    if D % group_size or (D * bits) % 32:
        raise ValueError("D must be a multiple of group_size and of 32/bits")
    rows = x.size // D
    codes = np.zeros(x.shape[:-1] + (D * bits // 32,), np.uint32)
    scales = np.zeros(x.shape[:-1] + (D // group_size,), _NP_STORAGE[scale_dtype])
    biases = np.zeros_like(scales)
    lib().orc_quantize_affine(_ptr(x), DTYPE_CODE[dtype], rows, D, bits, group_size,
                              DTYPE_CODE[scale_dtype], _ptr(codes), _ptr(scales), _ptr(biases))
    return codes, scales, biases


def dequant_affine(codes, scales, biases, scale_dtype: str, bits: int, group_size: int):
    codes = _c(codes, np.uint32)
    scales = _c(scales, _NP_STORAGE[scale_dtype])
    biases = _c(biases, _NP_STORAGE[scale_dtype])
    D = codes.shape[-1] * 32 // bits
    rows = codes.size // codes.shape[-1]
    out = np.zeros(codes.shape[:-1] + (D,), np.float32)
    lib().orc_dequant_affine(_ptr(codes), _ptr(scales), _ptr(biases), DTYPE_CODE[scale_dtype],
                             rows, D, bits, group_size, _ptr(out))
    return out


def quantize_q8_0(x: np.ndarray, dtype: str):
    """Q8_0 quantize the last axis.  Returns (codes int8, d fp16 bit patterns)."""
    x = _c(x, _NP_STORAGE[dtype])
    D = x.shape[-1]
    if D % 32:
        raise ValueError("D must be a multiple of 32")
    rows = x.size // D
    codes = np.zeros(x.shape, np.int8)
    d = np.zeros(x.shape[:-1] + (D // 32,), np.uint16)
    lib().orc_quantize_q8_0(_ptr(x), DTYPE_CODE[dtype], rows, D, _ptr(codes), _ptr(d))
    return codes, d


def dequant_q8_0(codes, d):
    codes = _c(codes, np.int8)
    d = _c(d, np.uint16)
    D = codes.shape[-1]
    rows = codes.size // D
    out = np.zeros(codes.shape, np.float32)
    lib().orc_dequant_q8_0(_ptr(codes), _ptr(d), rows, D, _ptr(out))
    return out


def quantize_qsym(x: np.ndarray, dtype: str, bits: int):
    """Symmetric 32-blocks at 4 or 5 bits.  Returns (codes as uint32 words of
    the rows' bit streams, d fp16 bit patterns)."""
    x = _c(x, _NP_STORAGE[dtype])
    D = x.shape[-1]
    if D % 32 or (D * bits) % 32:
        raise ValueError("D must be a multiple of 32")
    rows = x.size // D
    codes = np.zeros(x.shape[:-1] + (D * bits // 32,), np.uint32)
    d = np.zeros(x.shape[:-1] + (D // 32,), np.uint16)
    lib().orc_quantize_qsym(_ptr(x), DTYPE_CODE[dtype], rows, D, bits, _ptr(codes), _ptr(d))
    return codes, d


def dequant_qsym(codes, d, bits: int):
    codes = _c(codes, np.uint32)
    d = _c(d, np.uint16)
    D = codes.shape[-1] * 32 // bits
    rows = codes.size // codes.shape[-1]
    out = np.zeros(codes.shape[:-1] + (D,), np.float32)
    lib().orc_dequant_qsym(_ptr(codes), _ptr(d), rows, D, bits, _ptr(out))
    return out


def quantize(x: np.ndarray, dtype: str, mode: str, bits: int = 8, group_size: int = 64,
             scale_dtype: str | None = None):
    """Uniform front end: returns dict(codes=..., scales=..., biases=... or None)."""
    if mode == "qsym":
        c, d = quantize_qsym(x, dtype, bits)
        return {"codes": c, "scales": d, "biases": None}
    if mode == "affine":
        c, s, b = quantize_affine(x, dtype, bits, group_size, scale_dtype)
        return {"codes": c, "scales": s, "biases": b}
    if mode == "q8_0":
        c, d = quantize_q8_0(x, dtype)
        return {"codes": c, "scales": d, "biases": None}
    raise ValueError(mode)


def dequant(pack: dict, mode: str, bits: int = 8, group_size: int = 64,
            scale_dtype: str = "f16") -> np.ndarray:
    if mode == "affine":
        return dequant_affine(pack["codes"], pack["scales"], pack["biases"], scale_dtype,
                              bits, group_size)
    if mode == "qsym":
        return dequant_qsym(pack["codes"], pack["scales"], bits)
    return dequant_q8_0(pack["codes"], pack["scales"])


def append_rows(cache: dict, new: np.ndarray, dtype: str, offset: int, mode: str,
                bits: int = 8, group_size: int = 64, scale_dtype: str | None = None) -> dict:
    """Quantize ``new`` [B,H,T,D] into rows [offset, offset+T) of a copy of
    ``cache`` (arrays [B,H,Lcap,.]); every other row is left as it was
    ([MLX-KVU] fast.cpp kv_update / quantized.h kv_update: the new token's K
    and V rows are quantized into the cache at the offset)."""
    T = new.shape[2]
    q = quantize(new, dtype, mode, bits, group_size, scale_dtype)
    out = {}
    for name, arr in cache.items():
        if arr is None:
            out[name] = None
            continue
        a = arr.copy()
        a[:, :, offset:offset + T] = q[name]
        out[name] = a
    return out


# --------------------------------------------------------------------------- attention
def attention(q32: np.ndarray, khat: np.ndarray, vhat: np.ndarray, scale: float,
              mask: np.ndarray | None = None, causal: bool = False) -> np.ndarray:
    """softmax(scale * q K^T + mask) V in fp64 on dequantized fp32 K^, V^.

    q32: [B,Hq,Lq,D] fp32; khat, vhat: [B,Hk,L,D] fp32; mask: fp32,
    broadcastable to [B,Hq,Lq,L] (additive).  Returns fp64 [B,Hq,Lq,D]."""
    q32 = _c(q32, np.float32)
    khat = _c(khat, np.float32)
    vhat = _c(vhat, np.float32)
    B, Hq, Lq, D = q32.shape
    _, Hk, L, _ = khat.shape
    if Hq % Hk:
        raise ValueError("Hq must be a multiple of Hk")
    out = np.zeros((B, Hq, Lq, D), np.float64)
    mptr, sptr, mbuf = None, None, None
    if mask is not None:
        mbuf = np.asarray(mask, np.float32)
        while mbuf.ndim < 4:
            mbuf = mbuf[None]
        mbuf = np.broadcast_to(mbuf, (B, Hq, Lq, L))
        sptr = np.array([s // 4 if n > 1 else 0 for s, n in zip(mbuf.strides, mbuf.shape)],
                        np.int64)
        mptr = ctypes.c_void_p(mbuf.__array_interface__["data"][0])
    lib().orc_attention(_ptr(q32), _ptr(khat), _ptr(vhat), B, Hq, Hk, Lq, L, D, float(scale),
                        mptr, None if sptr is None else _ptr(sptr), int(bool(causal)), _ptr(out))
    return out
