"""Torch-facing binding of libqkv.so.

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the HIP stream, and a status other than QKV_OK raises
:class:`QKVError`.  Every step of quantization and attention runs in the HIP
kernels behind the C ABI; there is no CPU path.

The function names are those of the C ABI (include/qkv.h):
``qkv_quantize``, ``qkv_update_append``, ``qsdpa_workspace_bytes``,
``qsdpa_workspace_reset``, ``qsdpa_plan``, ``qsdpa_decode``,
``qsdpa_decode_static``, ``qsdpa_decode_append``, ``qsdpa_prefill``,
``qkv_dequantize``.
"""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from . import _lib
from ._lib import QKVError  # noqa: F401

_DT = {torch.float32: _lib.QKV_F32, torch.float16: _lib.QKV_F16, torch.bfloat16: _lib.QKV_BF16}
_DT_NAME = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_ALGO = {"auto": _lib.QKV_ALGO_AUTO, "generic": _lib.QKV_ALGO_GENERIC,
         "matrix": _lib.QKV_ALGO_MATRIX, "unfused": _lib.QKV_ALGO_UNFUSED,
         "dequant_f16": _lib.QKV_ALGO_DEQUANT_F16}


def torch_dtype(name_or_dtype) -> torch.dtype:
    if isinstance(name_or_dtype, torch.dtype):
        return name_or_dtype
    return _DT_NAME[name_or_dtype]


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@dataclasses.dataclass
class Pack:
    """A quantized K or V cache: codes, scales and (affine) biases, each
    [B, H, L_cap, *] with rows of one token of one head."""
    mode: str                      # "affine" | "q8_0" | "qsym" | "dense"
    bits: int
    group_size: int
    D: int
    codes: torch.Tensor            # affine, qsym: int32 words [B,H,L_cap,D*bits/32] (each row's
                                   # least-significant-first code stream); q8_0: int8 [B,H,L_cap,D];
                                   # dense: fp16 values [B,H,L_cap,D]
    scales: torch.Tensor | None    # [B,H,L_cap,D/group_size] (None for dense)
    biases: torch.Tensor | None    # affine only

    @property
    def B(self) -> int:
        return self.codes.shape[0]

    @property
    def H(self) -> int:
        return self.codes.shape[1]

    @property
    def L_cap(self) -> int:
        return self.codes.shape[2]

    @property
    def scale_dtype(self) -> torch.dtype:
        return self.codes.dtype if self.scales is None else self.scales.dtype

    def c_struct(self) -> _lib.QkvPack:
        c, s = self.codes, self.scales
        if self.mode == "dense":
            if c.stride(3) != 1 or any(c.stride(i) % c.shape[3] for i in range(3)):
                raise ValueError("pack rows must be contiguous, strides whole rows")
            rs = [c.stride(i) // c.shape[3] for i in range(3)]
            return _lib.QkvPack(mode=_lib.QKV_DENSE, bits=16, group_size=self.D,
                                scale_dtype=_dt(c), B=c.shape[0], H=c.shape[1], L_cap=c.shape[2],
                                D=self.D, codes=c.data_ptr(), scales=None, biases=None,
                                stride_b=rs[0], stride_h=rs[1], stride_l=rs[2])
        if c.stride(3) != 1 or s.stride(3) != 1:
            raise ValueError("pack rows must be contiguous")
        if self.biases is not None and self.biases.stride() != s.stride():
            raise ValueError("biases must have the layout of scales")
        if any(c.stride(i) % c.shape[3] or s.stride(i) % s.shape[3] for i in range(3)):
            raise ValueError("pack strides must be whole rows")
        rs = [c.stride(i) // c.shape[3] for i in range(3)]
        ss = [s.stride(i) // s.shape[3] for i in range(3)]
        if rs != ss:
            raise ValueError("codes and scales must share row strides")
        return _lib.QkvPack(
            mode={"affine": _lib.QKV_AFFINE, "q8_0": _lib.QKV_Q8_0, "qsym": _lib.QKV_QSYM}[self.mode],
            bits=self.bits, group_size=self.group_size, scale_dtype=_dt(s),
            B=c.shape[0], H=c.shape[1], L_cap=c.shape[2], D=self.D,
            codes=c.data_ptr(), scales=s.data_ptr(),
            biases=None if self.biases is None else self.biases.data_ptr(),
            stride_b=rs[0], stride_h=rs[1], stride_l=rs[2])


def empty_pack(B: int, H: int, L_cap: int, D: int, mode: str = "affine", bits: int = 4,
               group_size: int = 64, dtype=torch.float16, device="cuda") -> Pack:
    """Allocate a zero-filled dense pack (the caller owns the memory)."""
    dtype = torch_dtype(dtype)
    if mode == "dense":
        return Pack("dense", 16, D, D, torch.zeros((B, H, L_cap, D), dtype=torch.float16, device=device),
                    None, None)
    if mode == "qsym":
        return Pack("qsym", bits, 32, D,
                    torch.zeros((B, H, L_cap, D * bits // 32), dtype=torch.int32, device=device),
                    torch.zeros((B, H, L_cap, D // 32), dtype=torch.float16, device=device), None)
    if mode == "q8_0":
        return Pack("q8_0", 8, 32, D,
                    torch.zeros((B, H, L_cap, D), dtype=torch.int8, device=device),
                    torch.zeros((B, H, L_cap, D // 32), dtype=torch.float16, device=device), None)
    if mode != "affine":
        raise ValueError(mode)
    return Pack("affine", bits, group_size, D,
                torch.zeros((B, H, L_cap, D * bits // 32), dtype=torch.int32, device=device),
                torch.zeros((B, H, L_cap, D // group_size), dtype=dtype, device=device),
                torch.zeros((B, H, L_cap, D // group_size), dtype=dtype, device=device))


def _src_strides(x: torch.Tensor):
    if x.dim() != 4 or x.stride(3) != 1:
        raise ValueError("source must be [B,H,L,D] with D contiguous")
    return _lib.i64_array([x.stride(0), x.stride(1), x.stride(2)])


def qkv_quantize(x: torch.Tensor, mode: str = "affine", bits: int = 4, group_size: int = 64,
                 L_cap: int | None = None, out: Pack | None = None) -> Pack:
    """Quantize x[B,H,L,D] into rows [0, L) of a pack (a new one of capacity
    L_cap unless ``out`` is given)."""
    B, H, L, D = x.shape
    if out is None:
        out = empty_pack(B, H, L_cap or L, D, mode, bits, group_size, x.dtype, x.device)
    st = _lib.load().qkv_quantize(_ptr(x), _dt(x), _src_strides(x), L,
                                  ctypes.byref(out.c_struct()), _stream(x.device))
    _lib.check(st)
    return out


def qkv_update_append(k_cache: Pack, v_cache: Pack, k_new: torch.Tensor, v_new: torch.Tensor,
                      offset: int) -> None:
    """Quantize k_new/v_new [B,H,T,D] into rows [offset, offset+T) in place."""
    if k_new.shape != v_new.shape or k_new.stride() != v_new.stride() or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must share shape, strides and dtype")
    st = _lib.load().qkv_update_append(_ptr(k_new), _ptr(v_new), _dt(k_new), _src_strides(k_new),
                                       k_new.shape[2], offset, ctypes.byref(k_cache.c_struct()),
                                       ctypes.byref(v_cache.c_struct()), _stream(k_new.device))
    _lib.check(st)


def qkv_dequantize(src: Pack, L: int | None = None, out: Pack | None = None) -> Pack:
    """Rows [0, L) of a quantized pack as a dense fp16 pack (a new one of the
    source's capacity unless ``out`` is given)."""
    L = src.L_cap if L is None else L
    if out is None:
        out = empty_pack(src.B, src.H, src.L_cap, src.D, "dense", device=src.codes.device)
    st = _lib.load().qkv_dequantize(ctypes.byref(src.c_struct()), L, ctypes.byref(out.c_struct()),
                                    _stream(src.codes.device))
    _lib.check(st)
    return out


def _opts(num_splits: int, algo: str):
    return _lib.QkvAttnOpts(num_splits=int(num_splits), algo=_ALGO[algo])


def qsdpa_workspace_bytes(q: torch.Tensor, k: Pack, L: int, num_splits: int = 0,
                          algo: str = "auto") -> int:
    B, Hq, Lq, D = q.shape
    return int(_lib.load().qsdpa_workspace_bytes(B, Hq, Lq, D, L, ctypes.byref(k.c_struct()),
                                                 _dt(q), ctypes.byref(_opts(num_splits, algo))))


# kernel names of qsdpa_plan()["kernel"] (the device function names)
KERNEL_NAMES = {0: "attn_generic_kernel", 1: "attn_matrix_decode", 2: "attn_decode_narrow",
                3: "attn_matrix_prefill", 4: "unfused_scores_kernel", 5: "attn_decode_stream"}


def qsdpa_plan(q: torch.Tensor, k: Pack, L: int, num_splits: int = 0,
               algo: str = "auto") -> dict:
    """The launch plan of an attention call: kernel, splits, row tile, workspace."""
    B, Hq, Lq, D = q.shape
    pl = _lib.QkvAttnPlan()
    st = _lib.load().qsdpa_plan(B, Hq, Lq, D, L, ctypes.byref(k.c_struct()), _dt(q),
                                ctypes.byref(_opts(num_splits, algo)), ctypes.byref(pl))
    _lib.check(st)
    return {"algo": {1: "generic", 2: "matrix", 3: "unfused", 4: "dequant_f16"}[pl.algo], "num_splits": pl.num_splits,
            "row_tile": pl.row_tile, "keys_per_split": pl.keys_per_split,
            "workspace_bytes": pl.workspace_bytes, "kernel": KERNEL_NAMES[pl.kernel]}


class Workspace:
    """Reusable attention workspace (grows on demand): one buffer per (device,
    stream), so that calls on different streams never share split states or
    merge tickets.  Buffers start zero-filled (the ticket header at their
    start must; every call that completes leaves it zero)."""

    def __init__(self):
        self._buf: dict[tuple, torch.Tensor] = {}

    @staticmethod
    def _key(device, stream):
        device = torch.device(device)
        if stream is None:
            stream = torch.cuda.current_stream(device)
        return device, int(stream.cuda_stream)

    def get(self, nbytes: int, device, stream=None) -> torch.Tensor | None:
        """The buffer of (device, stream) with at least nbytes (None for 0);
        stream defaults to the device's current torch stream."""
        if nbytes == 0:
            return None
        key = self._key(device, stream)
        buf = self._buf.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(((nbytes + 255) // 256) * 256, dtype=torch.uint8, device=key[0])
            self._buf[key] = buf
        return buf

    def reset(self, device, stream=None) -> None:
        """Zero the ticket header of the (device, stream) buffer on that
        stream (qsdpa_workspace_reset), e.g. after a call that did not
        complete."""
        buf = self._buf.get(self._key(device, stream))
        if buf is not None:
            qsdpa_workspace_reset(buf, stream)


def qsdpa_workspace_reset(buf: torch.Tensor, stream=None) -> None:
    """Zero-fill the ticket header of a workspace buffer on its device's
    current (or the given) stream."""
    if stream is None:
        stream = torch.cuda.current_stream(buf.device)
    st = _lib.load().qsdpa_workspace_reset(_ptr(buf), buf.numel() * buf.element_size(),
                                           ctypes.c_void_p(stream.cuda_stream))
    _lib.check(st)


_default_ws = Workspace()


def _mask_args(mask: torch.Tensor | None, shape4):
    if mask is None:
        return None, 0, None
    m = mask
    while m.dim() < 4:
        m = m.unsqueeze(0)
    m = m.expand(*shape4)
    strides = [0 if n == 1 else s for s, n in zip(m.stride(), m.shape)]
    return _ptr(m), _dt(m), _lib.i64_array(strides)


def _attn_common(q, k, v, num_splits, algo, workspace, L):
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B,Hq,Lq,D] tensor")
    ws = workspace or _default_ws
    nbytes = qsdpa_workspace_bytes(q, k, L, num_splits, algo)
    buf = ws.get(nbytes, q.device)
    return buf, nbytes


def qsdpa_decode(q: torch.Tensor, k: Pack, v: Pack, L: int, scale: float,
                 mask: torch.Tensor | None = None, num_splits: int = 0, algo: str = "auto",
                 out: torch.Tensor | None = None, workspace: Workspace | None = None) -> torch.Tensor:
    """softmax(scale q K^T + mask) V for q[B,Hq,1,D] over keys [0, L)."""
    B, Hq, Lq, D = q.shape
    if Lq != 1:
        raise ValueError("decode takes one query per head")
    out = torch.empty_like(q) if out is None else out
    buf, nbytes = _attn_common(q, k, v, num_splits, algo, workspace, L)
    mp, mdt, ms = _mask_args(mask, (B, Hq, 1, L))
    st = _lib.load().qsdpa_decode(_ptr(q), _dt(q), B, Hq, D, ctypes.byref(k.c_struct()),
                                  ctypes.byref(v.c_struct()), L, float(scale), mp, mdt, ms,
                                  _ptr(out), _ptr(buf), nbytes,
                                  ctypes.byref(_opts(num_splits, algo)), _stream(q.device))
    _lib.check(st)
    return out


def qsdpa_decode_append(q: torch.Tensor, k: Pack, v: Pack, k_new: torch.Tensor, v_new: torch.Tensor,
                        offset: int, scale: float, mask: torch.Tensor | None = None,
                        num_splits: int = 0, algo: str = "auto", out: torch.Tensor | None = None,
                        workspace: Workspace | None = None) -> torch.Tensor:
    """One decoding step: k_new/v_new [B,Hk,1,D] (q's dtype) quantized into
    row ``offset`` of the packs, then softmax(scale q K^T + mask) V over keys
    [0, offset + 1) -- qkv_update_append followed by qsdpa_decode, as one
    launch where the narrow decode kernel takes the call."""
    B, Hq, Lq, D = q.shape
    if Lq != 1:
        raise ValueError("decode takes one query per head")
    if k_new.shape != v_new.shape or k_new.stride() != v_new.stride() or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must share shape, strides and dtype")
    if k_new.shape[2] != 1:
        raise ValueError("a decode step appends one token per (batch, kv head)")
    L = offset + 1
    out = torch.empty_like(q) if out is None else out
    buf, nbytes = _attn_common(q, k, v, num_splits, algo, workspace, L)
    mp, mdt, ms = _mask_args(mask, (B, Hq, 1, L))
    st = _lib.load().qsdpa_decode_append(_ptr(q), _dt(q), B, Hq, D, _ptr(k_new), _ptr(v_new),
                                         _src_strides(k_new), offset, ctypes.byref(k.c_struct()),
                                         ctypes.byref(v.c_struct()), float(scale), mp, mdt, ms,
                                         _ptr(out), _ptr(buf), nbytes,
                                         ctypes.byref(_opts(num_splits, algo)), _stream(q.device))
    _lib.check(st)
    return out


def qsdpa_decode_static(q: torch.Tensor, k: Pack, v: Pack, L: int, scale: float,
                        mask: torch.Tensor | None = None, num_splits: int = 0,
                        algo: str = "auto", out: torch.Tensor | None = None) -> torch.Tensor:
    """qsdpa_decode with the library's static per-GPU workspace: the call
    itself allocates nothing (``out`` given).  Calls that overlap on one GPU
    race on that workspace."""
    B, Hq, Lq, D = q.shape
    if Lq != 1:
        raise ValueError("decode takes one query per head")
    if q.dim() != 4 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B,Hq,1,D] tensor")
    out = torch.empty_like(q) if out is None else out
    mp, mdt, ms = _mask_args(mask, (B, Hq, 1, L))
    st = _lib.load().qsdpa_decode_static(_ptr(q), _dt(q), B, Hq, D, ctypes.byref(k.c_struct()),
                                         ctypes.byref(v.c_struct()), L, float(scale), mp, mdt, ms,
                                         _ptr(out), ctypes.byref(_opts(num_splits, algo)),
                                         _stream(q.device))
    _lib.check(st)
    return out


def qsdpa_prefill(q: torch.Tensor, k: Pack, v: Pack, L: int, scale: float, causal: bool = False,
                  mask: torch.Tensor | None = None, num_splits: int = 0, algo: str = "auto",
                  out: torch.Tensor | None = None,
                  workspace: Workspace | None = None) -> torch.Tensor:
    """softmax(scale q K^T + mask) V for q[B,Hq,Lq,D] over keys [0, L); causal
    hides key j from query i when j > L - Lq + i."""
    B, Hq, Lq, D = q.shape
    if causal and mask is not None:
        raise ValueError("pass either causal=True or an additive mask")
    out = torch.empty_like(q) if out is None else out
    buf, nbytes = _attn_common(q, k, v, num_splits, algo, workspace, L)
    kind = _lib.QKV_MASK_CAUSAL if causal else (_lib.QKV_MASK_ADDITIVE if mask is not None
                                                else _lib.QKV_MASK_NONE)
    mp, mdt, ms = _mask_args(mask, (B, Hq, Lq, L))
    st = _lib.load().qsdpa_prefill(_ptr(q), _dt(q), B, Hq, Lq, D, ctypes.byref(k.c_struct()),
                                   ctypes.byref(v.c_struct()), L, float(scale), kind, mp, mdt, ms,
                                   _ptr(out), _ptr(buf), nbytes,
                                   ctypes.byref(_opts(num_splits, algo)), _stream(q.device))
    _lib.check(st)
    return out


class PreparedQuantize:
    """A qkv_quantize call with its arguments marshalled once: calling it
    quantizes the same x[B,H,L,D] into rows [0, L) of the same pack."""

    def __init__(self, x: torch.Tensor, out: Pack):
        self._keep = (x, out)
        self._c = out.c_struct()
        self._fn = _lib.load().qkv_quantize
        self._args = (_ptr(x), _dt(x), _src_strides(x), x.shape[2], ctypes.byref(self._c), _stream(x.device))

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st:
            _lib.check(st)


class PreparedAppend:
    """A qkv_update_append call with its arguments marshalled once; calling it
    with an offset quantizes the same k_new/v_new into rows [offset, offset+T)."""

    def __init__(self, k_cache: Pack, v_cache: Pack, k_new: torch.Tensor, v_new: torch.Tensor):
        if k_new.shape != v_new.shape or k_new.stride() != v_new.stride() or k_new.dtype != v_new.dtype:
            raise ValueError("k_new and v_new must share shape, strides and dtype")
        self._keep = (k_cache, v_cache, k_new, v_new)
        self._kc, self._vc = k_cache.c_struct(), v_cache.c_struct()
        self._strides = _src_strides(k_new)
        self._fn = _lib.load().qkv_update_append
        self._head = (_ptr(k_new), _ptr(v_new), _dt(k_new), self._strides, k_new.shape[2])
        self._tail = (ctypes.byref(self._kc), ctypes.byref(self._vc), _stream(k_new.device))

    def __call__(self, offset: int) -> None:
        st = self._fn(*self._head, offset, *self._tail)
        if st:
            _lib.check(st)


class PreparedAttention:
    """A qsdpa_decode (q[B,Hq,1,D], no causal mask) or qsdpa_prefill call with
    its arguments marshalled once.

    Calling the object re-issues the same launch (same tensors, same stream)
    with only the ctypes call on the host path -- the form a serving loop or
    a benchmark uses.  The tensors must stay alive and keep their storage."""

    def __init__(self, q: torch.Tensor, k: Pack, v: Pack, L: int, scale: float,
                 out: torch.Tensor, mask: torch.Tensor | None = None, causal: bool = False,
                 num_splits: int = 0, algo: str = "auto", workspace: Workspace | None = None):
        B, Hq, Lq, D = q.shape
        if not q.is_contiguous() or out.shape != q.shape or not out.is_contiguous():
            raise ValueError("attention takes contiguous q, out of one shape [B,Hq,Lq,D]")
        if causal and mask is not None:
            raise ValueError("pass either causal=True or an additive mask")
        buf, nbytes = _attn_common(q, k, v, num_splits, algo, workspace, L)
        mp, mdt, ms = _mask_args(mask, (B, Hq, Lq, L))
        self._keep = (q, k, v, out, buf, mask)
        self._kc, self._vc = k.c_struct(), v.c_struct()
        self._opts = _opts(num_splits, algo)
        L_ = _lib.load()
        head = (_ptr(q), _dt(q), B, Hq)
        tail = (ctypes.byref(self._kc), ctypes.byref(self._vc), L, float(scale))
        rest = (_ptr(out), _ptr(buf), nbytes, ctypes.byref(self._opts), _stream(q.device))
        if Lq == 1 and not causal:
            self._fn = L_.qsdpa_decode
            self._args = head + (D,) + tail + (mp, mdt, ms) + rest
        else:
            kind = _lib.QKV_MASK_CAUSAL if causal else (
                _lib.QKV_MASK_ADDITIVE if mask is not None else _lib.QKV_MASK_NONE)
            self._fn = L_.qsdpa_prefill
            self._args = head + (Lq, D) + tail + (kind, mp, mdt, ms) + rest
        self.out = out

    def set_timing(self, begin: torch.cuda.Event | None, end: torch.cuda.Event | None) -> None:
        """Have later calls record `begin` / `end` (timing-enabled events that
        have been recorded once, so that their HIP handles exist) around the
        attention kernel alone; None stops it."""
        if begin is None or end is None:
            self._opts.timing_events[0] = self._opts.timing_events[1] = None
            return
        self._opts.timing_events[0] = begin.cuda_event
        self._opts.timing_events[1] = end.cuda_event

    def __call__(self) -> torch.Tensor:
        st = self._fn(*self._args)
        if st:
            _lib.check(st)
        return self.out


class PreparedDecodeAppend:
    """A qsdpa_decode_append call (no mask) with its arguments marshalled
    once: calling it appends the same k_new/v_new at the same offset and
    attends keys [0, offset + 1).  The tensors must stay alive."""

    def __init__(self, q: torch.Tensor, k: Pack, v: Pack, k_new: torch.Tensor, v_new: torch.Tensor,
                 offset: int, scale: float, out: torch.Tensor, num_splits: int = 0, algo: str = "auto",
                 workspace: Workspace | None = None):
        B, Hq, Lq, D = q.shape
        if Lq != 1 or not q.is_contiguous() or out.shape != q.shape or not out.is_contiguous():
            raise ValueError("decode with append takes contiguous q, out of one shape [B,Hq,1,D]")
        if k_new.shape != v_new.shape or k_new.stride() != v_new.stride() or k_new.dtype != v_new.dtype:
            raise ValueError("k_new and v_new must share shape, strides and dtype")
        buf, nbytes = _attn_common(q, k, v, num_splits, algo, workspace, offset + 1)
        self._keep = (q, k, v, k_new, v_new, out, buf)
        self._kc, self._vc = k.c_struct(), v.c_struct()
        self._opts = _opts(num_splits, algo)
        self._strides = _src_strides(k_new)
        self._fn = _lib.load().qsdpa_decode_append
        self._args = (_ptr(q), _dt(q), B, Hq, D, _ptr(k_new), _ptr(v_new), self._strides, offset,
                      ctypes.byref(self._kc), ctypes.byref(self._vc), float(scale), None, 0, None,
                      _ptr(out), _ptr(buf), nbytes, ctypes.byref(self._opts), _stream(q.device))
        self.out = out

    def set_timing(self, begin: torch.cuda.Event | None, end: torch.cuda.Event | None) -> None:
        """As PreparedAttention.set_timing: events around the attention kernel."""
        if begin is None or end is None:
            self._opts.timing_events[0] = self._opts.timing_events[1] = None
            return
        self._opts.timing_events[0] = begin.cuda_event
        self._opts.timing_events[1] = end.cuda_event

    def __call__(self) -> torch.Tensor:
        st = self._fn(*self._args)
        if st:
            _lib.check(st)
        return self.out


class PreparedDecode(PreparedAttention):
    """PreparedAttention restricted to decode shapes (q[B,Hq,1,D])."""

    def __init__(self, q: torch.Tensor, k: Pack, v: Pack, L: int, scale: float,
                 out: torch.Tensor, mask: torch.Tensor | None = None, num_splits: int = 0,
                 algo: str = "auto", workspace: Workspace | None = None):
        if q.dim() != 4 or q.shape[2] != 1:
            raise ValueError("decode takes contiguous q, out of shape [B,Hq,1,D]")
        super().__init__(q, k, v, L, scale, out, mask=mask, num_splits=num_splits, algo=algo,
                         workspace=workspace)
