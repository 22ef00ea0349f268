"""Attention over a group-quantized KV cache, native to AMD Instinct MI355X.

The compute path is libqkv.so (hand-written HIP kernels for gfx950 behind the
C ABI in include/qkv.h); this package is its torch-facing binding.
"""
from .api import (Pack, PreparedAppend, PreparedAttention, PreparedDecode, PreparedDecodeAppend, PreparedQuantize,
                  QKVError,
                  Workspace,
                  empty_pack, qkv_dequantize, qkv_quantize, qkv_update_append, qsdpa_decode,
                  qsdpa_decode_append, qsdpa_decode_static, qsdpa_plan, qsdpa_prefill, qsdpa_workspace_bytes, qsdpa_workspace_reset, torch_dtype)

__all__ = ["Pack", "PreparedAppend", "PreparedAttention", "PreparedDecode", "PreparedDecodeAppend", "PreparedQuantize",
           "QKVError",
           "Workspace",
           "empty_pack", "qkv_dequantize", "qkv_quantize", "qkv_update_append", "qsdpa_decode",
           "qsdpa_decode_append", "qsdpa_decode_static", "qsdpa_plan",
           "qsdpa_prefill", "qsdpa_workspace_bytes", "qsdpa_workspace_reset", "torch_dtype"]
