"""The wider format set on the GPU: affine codes of 2, 3, 5 and 6 bits, head
size 96, and the symmetric 4/5-bit blocks (the Q4_0/Q5_0 reading), plus Q8_0
and affine 4/8-bit at head size 96.  Quantize and append must give the
oracle's bits; decode and prefill (on the generic kernel, with key splits
and the merge kernels; with fp16 queries and at most 4 heads per kv head the
decode also runs on the bit-stream decode kernel, or for the symmetric 4-bit
blocks at D 64 or 128 on the narrow matrix-core decode) must be within the
attention tolerance of the oracle."""
import math
import zlib

import numpy as np
import pytest
import torch

import quantized_kv_cache_amd as qkv
from tests._cases import (W, assert_close, assert_pack_equal, oracle_attention, oracle_pack,
                          pack_numpy, to_dev)

pytestmark = pytest.mark.gpu

FORMATS = [
    # mode, bits, gs, D, dtype
    ("affine", 2, 32, 128, "f16"),
    ("affine", 3, 64, 128, "f16"),
    ("affine", 3, 32, 96, "bf16"),
    ("affine", 5, 32, 256, "f16"),
    ("affine", 5, 128, 128, "f32"),
    ("affine", 6, 64, 64, "f16"),
    ("affine", 6, 32, 96, "f16"),
    ("affine", 2, 64, 256, "bf16"),
    ("affine", 4, 32, 96, "f16"),
    ("affine", 8, 32, 96, "f32"),
    ("q8_0", 8, 32, 96, "f16"),
    ("qsym", 4, 32, 128, "f16"),
    ("qsym", 5, 32, 96, "f16"),
    ("qsym", 4, 32, 256, "bf16"),
    ("qsym", 5, 32, 64, "f32"),
]


def _seed(*a):
    return zlib.crc32(repr(a).encode()) % 100000


def _case(fmt, B, Hq, Hk, Lq, L, dist="normal"):
    mode, bits, gs, D, dt = fmt
    s = _seed(fmt, B, Hq, Hk, Lq, L)
    q = W.random_case(s, (B, Hq, Lq, D), dist, dt)
    k = W.random_case(s + 1, (B, Hk, L, D), dist, dt)
    v = W.random_case(s + 2, (B, Hk, L, D), dist, dt)
    kp = qkv.qkv_quantize(to_dev(k, dt), mode, bits, gs)
    vp = qkv.qkv_quantize(to_dev(v, dt), mode, bits, gs)
    kr, vr = oracle_pack(k, dt, mode, bits, gs), oracle_pack(v, dt, mode, bits, gs)
    assert_pack_equal(pack_numpy(kp), kr)
    assert_pack_equal(pack_numpy(vp), vr)
    return q, kp, vp, kr, vr


@pytest.mark.parametrize("fmt", FORMATS, ids=lambda f: "-".join(map(str, f)))
def test_formats_quantize_append_and_decode(fmt):
    mode, bits, gs, D, dt = fmt
    q, kp, vp, kr, vr = _case(fmt, 2, 8, 2, 1, 517)
    scale = 1.0 / math.sqrt(D)
    ref = oracle_attention(q, dt, kr, vr, 517, mode, bits, gs, scale)
    qd = to_dev(q, dt)
    narrow = mode == "qsym" and bits == 4 and D in (64, 128) and dt == "f16"
    expect = "attn_decode_narrow" if narrow else "attn_decode_stream" if dt == "f16" else "attn_generic_kernel"
    assert qkv.qsdpa_plan(qd, kp, 517)["kernel"] == expect
    assert qkv.qsdpa_plan(qd, kp, 517, algo="generic")["kernel"] == "attn_generic_kernel"
    for algo in (("auto", "generic") if dt == "f16" else ("auto",)):
        for splits in (0, 1, 5, 17):
            out = qkv.qsdpa_decode(qd, kp, vp, 517, scale, num_splits=splits, algo=algo)
            assert_close(out, ref, f"decode {fmt} {algo} splits={splits}")
    # append three tokens at an offset: bit-exact rows, the rest untouched
    new_k = W.random_case(_seed(fmt, "k"), (2, 2, 3, D), "normal", dt)
    new_v = W.random_case(_seed(fmt, "v"), (2, 2, 3, D), "normal", dt)
    before_k = pack_numpy(kp)
    qkv.qkv_update_append(kp, vp, to_dev(new_k, dt), to_dev(new_v, dt), 200)
    after_k = pack_numpy(kp)
    nk = oracle_pack(new_k, dt, mode, bits, gs)
    for name, a in nk.items():
        if a is None:
            continue
        g, r = after_k[name][:, :, 200:203], a
        assert np.array_equal(np.ascontiguousarray(g).view(np.uint8), np.ascontiguousarray(r).view(np.uint8)), name
        keep = np.r_[0:200, 203:517]
        assert np.array_equal(np.ascontiguousarray(after_k[name][:, :, keep]).view(np.uint8),
                              np.ascontiguousarray(before_k[name][:, :, keep]).view(np.uint8)), name


@pytest.mark.parametrize("fmt", FORMATS[::2], ids=lambda f: "-".join(map(str, f)))
def test_formats_prefill(fmt):
    mode, bits, gs, D, dt = fmt
    q, kp, vp, kr, vr = _case(fmt, 1, 8, 2, 21, 300)
    ref = oracle_attention(q, dt, kr, vr, 300, mode, bits, gs, 0.1, causal=True)
    for splits in (0, 3):
        out = qkv.qsdpa_prefill(to_dev(q, dt), kp, vp, 300, 0.1, causal=True, num_splits=splits)
        assert_close(out, ref, f"prefill {fmt} splits={splits}")


def test_formats_rejected_by_matrix_only_algorithms():
    q, kp, vp, _, _ = _case(("affine", 3, 32, 128, "f16"), 1, 8, 2, 1, 100)
    for algo in ("matrix", "unfused", "dequant_f16"):
        with pytest.raises(qkv.QKVError):
            qkv.qsdpa_decode(to_dev(q, "f16"), kp, vp, 100, 0.1, algo=algo)


@pytest.mark.parametrize("name", ["decode_64k_3bit_gqa4", "decode_64k_qsym4_gqa4", "decode_16k_d96_gqa4"])
def test_format_workload_full(name):
    w = W.WORKLOADS[name]
    print(f"[format] {name}", flush=True)
    inp = W.make_inputs(w)
    kp = qkv.qkv_quantize(to_dev(inp["k"], w.dtype), w.mode, w.bits, w.group_size)
    vp = qkv.qkv_quantize(to_dev(inp["v"], w.dtype), w.mode, w.bits, w.group_size)
    kr = oracle_pack(inp["k"], w.dtype, w.mode, w.bits, w.group_size)
    vr = oracle_pack(inp["v"], w.dtype, w.mode, w.bits, w.group_size)
    assert_pack_equal(pack_numpy(kp), kr)
    assert_pack_equal(pack_numpy(vp), vr)
    out = qkv.qsdpa_decode(to_dev(inp["q"], w.dtype), kp, vp, w.L, w.scale)
    ref = oracle_attention(inp["q"], w.dtype, kr, vr, w.L, w.mode, w.bits, w.group_size, w.scale)
    assert_close(out, ref, name, report=True)


# the symmetric 4-bit blocks on the narrow matrix-core decode: GQA factors 1-4,
# both head sizes, ragged lengths, an additive mask, split counts, and the
# same bits on a repeated call
QSYM_NARROW = [
    # B, Hq, Hk, D, L, mask
    (2, 8, 2, 128, 1000, False),
    (1, 3, 3, 64, 777, False),
    (1, 6, 2, 128, 4099, True),
    (2, 4, 2, 64, 130, False),
    (1, 32, 8, 128, 2113, True),
]


@pytest.mark.parametrize("case", QSYM_NARROW, ids=lambda c: "-".join(map(str, c)))
def test_qsym4_narrow_decode(case):
    B, Hq, Hk, D, L, use_mask = case
    fmt = ("qsym", 4, 32, D, "f16")
    q, kp, vp, kr, vr = _case(fmt, B, Hq, Hk, 1, L)
    scale = 1.0 / math.sqrt(D)
    mask = None
    if use_mask:
        rng = np.random.default_rng(_seed(case, "mask"))
        mask = np.where(rng.random((B, Hq, 1, L)) < 0.2, -np.inf, rng.normal(0, 1, (B, Hq, 1, L))).astype(np.float32)
        mask[..., 0] = 0.0                        # every row sees a key
    ref = oracle_attention(q, "f16", kr, vr, L, "qsym", 4, 32, scale, mask=mask)
    qd = to_dev(q, "f16")
    md = None if mask is None else to_dev(mask, "f32")
    assert qkv.qsdpa_plan(qd, kp, L)["kernel"] == "attn_decode_narrow"
    first = None
    for splits in (0, 1, 3, 9):
        out = qkv.qsdpa_decode(qd, kp, vp, L, scale, mask=md, num_splits=splits)
        assert_close(out, ref, f"qsym4 narrow {case} splits={splits}", report=splits == 0)
        if splits == 0:
            first = out.clone()
    again = qkv.qsdpa_decode(qd, kp, vp, L, scale, mask=md)
    assert torch.equal(again, first)


def _offset_scales(p):
    """The pack with its scale plane copied to storage 2 bytes past an aligned
    address (the symmetric formats only require 2-byte alignment)."""
    n = p.scales.numel()
    flat = torch.zeros(n + 8, dtype=p.scales.dtype, device=p.scales.device)
    view = flat[1:1 + n].view(p.scales.shape)
    view.copy_(p.scales)
    assert view.data_ptr() % 4 == 2
    return qkv.Pack(p.mode, p.bits, p.group_size, p.D, p.codes, view, None)


@pytest.mark.parametrize("D", [64, 128])
def test_qsym4_narrow_unaligned_scales(D):
    fmt = ("qsym", 4, 32, D, "f16")
    q, kp, vp, kr, vr = _case(fmt, 1, 8, 2, 1, 1500)
    qd = to_dev(q, "f16")
    scale = 1.0 / math.sqrt(D)
    ref = oracle_attention(q, "f16", kr, vr, 1500, "qsym", 4, 32, scale)
    aligned = qkv.qsdpa_decode(qd, kp, vp, 1500, scale)
    ku, vu = _offset_scales(kp), _offset_scales(vp)
    assert qkv.qsdpa_plan(qd, ku, 1500)["kernel"] == "attn_decode_narrow"
    out = qkv.qsdpa_decode(qd, ku, vu, 1500, scale)
    assert_close(out, ref, f"qsym4 narrow D={D}, 2-byte aligned scales")
    assert torch.equal(out, aligned)


# the bit-stream decode kernel: GQA factors 1-4, every head size, ragged
# lengths, an additive mask, split counts (one split writes the output itself,
# several go through the merge kernel), repeat bits
STREAM_CASES = [
    # mode, bits, gs, D, B, Hq, Hk, L, mask
    ("affine", 3, 64, 128, 1, 8, 2, 1999, False),
    ("affine", 2, 128, 256, 2, 3, 3, 700, True),
    ("affine", 5, 32, 96, 1, 8, 4, 333, False),
    ("affine", 6, 64, 64, 2, 4, 1, 4097, True),
    ("qsym", 5, 32, 128, 1, 32, 8, 1500, False),
    ("qsym", 4, 32, 96, 1, 6, 2, 64, False),
    ("q8_0", 8, 32, 96, 1, 4, 2, 1025, True),
    ("affine", 8, 32, 96, 1, 2, 2, 1, False),          # a single key
]


@pytest.mark.parametrize("case", STREAM_CASES, ids=lambda c: "-".join(map(str, c)))
def test_stream_decode(case):
    mode, bits, gs, D, B, Hq, Hk, L, use_mask = case
    fmt = (mode, bits, gs, D, "f16")
    q, kp, vp, kr, vr = _case(fmt, B, Hq, Hk, 1, L)
    scale = 1.0 / math.sqrt(D)
    mask = None
    if use_mask:
        rng = np.random.default_rng(_seed(case, "mask"))
        mask = np.where(rng.random((B, Hq, 1, L)) < 0.25, -np.inf, rng.normal(0, 1, (B, Hq, 1, L))).astype(np.float32)
        mask[..., L // 2] = 0.0                       # every row sees a key
        mask[0, 0, 0, :] = -np.inf                    # a fully masked row -> zeros
    ref = oracle_attention(q, "f16", kr, vr, L, mode, bits, gs, scale, mask=mask)
    qd = to_dev(q, "f16")
    md = None if mask is None else to_dev(mask, "f32")
    assert qkv.qsdpa_plan(qd, kp, L)["kernel"] == "attn_decode_stream"
    first = None
    for splits in (0, 1, 2, 7):
        out = qkv.qsdpa_decode(qd, kp, vp, L, scale, mask=md, num_splits=splits)
        assert_close(out, ref, f"stream decode {case} splits={splits}", report=splits == 0)
        if splits == 0:
            first = out.clone()
    assert torch.equal(qkv.qsdpa_decode(qd, kp, vp, L, scale, mask=md), first)
