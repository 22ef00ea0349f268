"""Shared helpers of the GPU parity tests: numpy <-> torch marshalling, the
oracle pipeline on the same seeded inputs, and the attention tolerance."""
from __future__ import annotations

import numpy as np
import torch

import oracle as orc
from quantized_kv_cache_amd import workloads as W

ATOL, RTOL = 2e-3, 1e-2     # |gpu - ref| <= ATOL + RTOL * |ref|

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_dev(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def from_dev(t: torch.Tensor) -> np.ndarray:
    """Storage view of a device tensor as numpy (bf16 -> uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def pack_numpy(p) -> dict:
    """A GPU Pack as the oracle's numpy dict (bit patterns preserved)."""
    out = {"codes": from_dev(p.codes), "scales": from_dev(p.scales),
           "biases": None if p.biases is None else from_dev(p.biases)}
    if p.mode == "q8_0":
        out["scales"] = out["scales"].view(np.uint16)
    return out


def oracle_pack(x: np.ndarray, dtype: str, mode: str, bits: int, gs: int) -> dict:
    pk = orc.quantize(x, dtype, mode, bits, gs)
    if mode == "q8_0":
        pk["scales"] = pk["scales"].view(np.uint16)
    return pk


_UINT = {1: np.uint8, 2: np.uint16, 4: np.uint32}


def assert_pack_equal(gpu: dict, ref: dict, rows=None):
    """Bit-exact comparison of codes, scales and biases."""
    for name in ("codes", "scales", "biases"):
        if ref[name] is None:
            assert gpu[name] is None
            continue
        g, r = gpu[name], ref[name]
        if rows is not None:
            g, r = g[:, :, rows], r[:, :, rows]
        g, r = np.ascontiguousarray(g), np.ascontiguousarray(r)
        assert g.shape == r.shape and g.dtype.itemsize == r.dtype.itemsize, name
        gu, ru = g.view(_UINT[g.dtype.itemsize]), r.view(_UINT[r.dtype.itemsize])
        if not np.array_equal(gu, ru):
            bad = np.argwhere(gu != ru)
            i = tuple(bad[0])
            raise AssertionError(f"{name}: {len(bad)} elements differ; first at {i}: "
                                 f"gpu={gu[i]:#x} oracle={ru[i]:#x}")


def dequant(pk: dict, mode: str, bits: int, gs: int, scale_dtype: str) -> np.ndarray:
    if mode == "q8_0":
        return orc.dequant_q8_0(pk["codes"], pk["scales"])
    if mode == "qsym":
        return orc.dequant_qsym(pk["codes"], pk["scales"], bits)
    return orc.dequant_affine(pk["codes"], pk["scales"], pk["biases"], scale_dtype, bits, gs)


def oracle_attention(q: np.ndarray, qdt: str, kp: dict, vp: dict, L: int, mode: str, bits: int,
                     gs: int, scale: float, mask=None, causal=False) -> np.ndarray:
    sdt = "f16" if mode in ("q8_0", "qsym") else qdt
    kh = dequant({k: (None if v is None else v[:, :, :L]) for k, v in kp.items()}, mode, bits, gs, sdt)
    vh = dequant({k: (None if v is None else v[:, :, :L]) for k, v in vp.items()}, mode, bits, gs, sdt)
    return orc.attention(orc.to_f32(q, qdt), kh, vh, scale, mask=mask, causal=causal)


def err_over_tol(gpu, ref: np.ndarray) -> float:
    """max |gpu - ref| / (ATOL + RTOL |ref|): below 1 passes, and how far
    below is the precision headroom."""
    g = gpu.detach().float().cpu().numpy().astype(np.float64) if isinstance(gpu, torch.Tensor) \
        else np.asarray(gpu, np.float64)
    return float(np.max(np.abs(g - ref) / (ATOL + RTOL * np.abs(ref))))


def assert_close(gpu: torch.Tensor, ref: np.ndarray, what: str = "", report: bool = False):
    g = gpu.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    tol = ATOL + RTOL * np.abs(ref)
    if report:
        print(f"[headroom] {what}: max err/tol = {float(np.max(err / tol)):.4f}, "
              f"max err = {float(err.max()):.3e}, output std = {float(ref.std()):.3e}", flush=True)
    if not np.all(err <= tol):
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {int((err > tol).sum())} of {err.size} outside tolerance; "
                             f"worst at {i}: gpu={g[i]!r} ref={ref[i]!r}")


def scale_dtype_of(mode: str, dtype: str) -> str:
    return "f16" if mode in ("q8_0", "qsym") else dtype


__all__ = ["ATOL", "RTOL", "TORCH_DT", "to_dev", "from_dev", "pack_numpy", "oracle_pack",
           "assert_pack_equal", "dequant", "oracle_attention", "assert_close", "err_over_tol",
           "scale_dtype_of",
           "W", "orc"]
