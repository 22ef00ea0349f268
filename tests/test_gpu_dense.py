"""Dense fp16 caches (the unquantized baseline the pages compare against) and
the dequantize-first strategy of the llama.cpp page (K/V dequantized into
dense fp16 copies, then dense matrix-core attention), against the oracle:

- qkv_dequantize gives fp16(the oracle's fp32 dequantized value), bit for bit;
- attention over dense packs (decode and prefill) is within the tolerance of
  the oracle's fp64 attention over the same fp16 values;
- algo="dequant_f16" over quantized packs is within the tolerance of the
  oracle's attention over its dequantized packs, including every row of the
  512-query Q8_0 prefill at full size."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_amd as qkv
from tests._cases import (W, assert_close, assert_pack_equal, dequant, oracle_attention,
                          oracle_pack, orc, pack_numpy, to_dev)

pytestmark = pytest.mark.gpu


def _dense_ref(q, k, v, dtype, scale, causal=False, mask=None):
    return orc.attention(orc.to_f32(q, dtype), orc.to_f32(k, dtype), orc.to_f32(v, dtype), scale,
                         mask=mask, causal=causal)


@pytest.mark.parametrize("mode,bits,gs,D", [("affine", 4, 64, 128), ("affine", 4, 32, 64),
                                            ("affine", 8, 128, 256), ("affine", 8, 64, 128),
                                            ("q8_0", 8, 32, 256), ("q8_0", 8, 32, 64)])
def test_dequantize_matches_oracle_bits(mode, bits, gs, D):
    B, H, L = 2, 3, 333
    x = W.random_case(17 + D + bits, (B, H, L, D), "normal", "f16")
    pk = qkv.qkv_quantize(to_dev(x, "f16"), mode, bits, gs, L_cap=L + 7)
    dense = qkv.qkv_dequantize(pk, L)
    ref = dequant(oracle_pack(x, "f16", mode, bits, gs), mode, bits, gs, "f16").astype(np.float16)
    got = dense.codes[:, :, :L].cpu().numpy()
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
    assert not dense.codes[:, :, L:].any()                      # rows past L untouched
    # into a strided destination (every second row of a larger buffer)
    big = qkv.empty_pack(B, H, 2 * L, D, "dense")
    view = qkv.Pack("dense", 16, D, D, big.codes[:, :, ::2], None, None)
    qkv.qkv_dequantize(pk, L, out=view)
    assert np.array_equal(big.codes[:, :, ::2].cpu().numpy().view(np.uint16), ref.view(np.uint16))
    assert not big.codes[:, :, 1::2].any()


def test_dense_quantize_and_append_store_the_values():
    x = W.random_case(3, (2, 2, 40, 128), "normal", "f16")
    pk = qkv.qkv_quantize(to_dev(x, "f16"), "dense", L_cap=50)
    assert np.array_equal(pk.codes[:, :, :40].cpu().numpy().view(np.uint16), x.view(np.uint16))
    vk = qkv.empty_pack(2, 2, 50, 128, "dense")
    new = W.random_case(4, (2, 2, 3, 128), "normal", "f16")
    qkv.qkv_update_append(pk, vk, to_dev(new, "f16"), to_dev(new, "f16"), 40)
    assert np.array_equal(pk.codes[:, :, 40:43].cpu().numpy().view(np.uint16), new.view(np.uint16))
    assert not pk.codes[:, :, 43:].any()


DENSE_CASES = [
    # B, Hq, Hk, Lq, L, D, causal
    (1, 32, 8, 1, 3000, 128, False),     # the 64K GQA-4 shape, short
    (1, 32, 2, 1, 2500, 256, False),     # the GQA-16 D256 shape, short
    (2, 8, 2, 1, 77, 64, False),
    (1, 16, 2, 40, 700, 128, True),      # prefill, 64-row tiles, ragged
    (1, 32, 2, 20, 1000, 256, True),     # prefill, 320 rows -> 128-row tiles
    (2, 4, 4, 9, 200, 64, False),
]


@pytest.mark.parametrize("case", DENSE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_dense_attention(case):
    B, Hq, Hk, Lq, L, D, causal = case
    q = W.random_case(50 + L, (B, Hq, Lq, D), "normal", "f16")
    k = W.random_case(51 + L, (B, Hk, L, D), "normal", "f16")
    v = W.random_case(52 + L, (B, Hk, L, D), "normal", "f16")
    kp = qkv.qkv_quantize(to_dev(k, "f16"), "dense")
    vp = qkv.qkv_quantize(to_dev(v, "f16"), "dense")
    qd = to_dev(q, "f16")
    scale = 1.0 / math.sqrt(D)
    assert qkv.qsdpa_plan(qd, kp, L)["kernel"] == "attn_matrix_prefill"
    ref = _dense_ref(q, k, v, "f16", scale, causal=causal)
    for splits in (0, 1, 3):
        if Lq == 1:
            out = qkv.qsdpa_decode(qd, kp, vp, L, scale, num_splits=splits)
        else:
            out = qkv.qsdpa_prefill(qd, kp, vp, L, scale, causal=causal, num_splits=splits)
        assert_close(out, ref, f"dense {case} splits={splits}")


PREPASS_CASES = [
    # dtype mode bits gs B Hq Hk Lq L D causal
    ("q8_0", 8, 32, 1, 32, 2, 40, 900, 256, True),
    ("q8_0", 8, 32, 1, 32, 2, 1, 2000, 256, False),
    ("affine", 4, 64, 1, 32, 8, 1, 3000, 128, False),
    ("affine", 8, 32, 2, 8, 2, 17, 300, 64, True),
    ("affine", 4, 128, 1, 16, 1, 70, 257, 128, False),
]


@pytest.mark.parametrize("case", PREPASS_CASES, ids=lambda c: "-".join(map(str, c)))
def test_dequantize_first_attention(case):
    mode, bits, gs, B, Hq, Hk, Lq, L, D, causal = case
    q = W.random_case(60 + L, (B, Hq, Lq, D), "normal", "f16")
    k = W.random_case(61 + L, (B, Hk, L + 5, D), "normal", "f16")
    v = W.random_case(62 + L, (B, Hk, L + 5, D), "normal", "f16")
    kp = qkv.qkv_quantize(to_dev(k, "f16"), mode, bits, gs)
    vp = qkv.qkv_quantize(to_dev(v, "f16"), mode, bits, gs)
    kr, vr = oracle_pack(k, "f16", mode, bits, gs), oracle_pack(v, "f16", mode, bits, gs)
    qd = to_dev(q, "f16")
    plan = qkv.qsdpa_plan(qd, kp, L, algo="dequant_f16")
    assert plan["algo"] == "dequant_f16" and plan["kernel"] == "attn_matrix_prefill"
    ref = oracle_attention(q, "f16", kr, vr, L, mode, bits, gs, 0.1, causal=causal)
    for splits in (0, 2):
        out = qkv.qsdpa_prefill(qd, kp, vp, L, 0.1, causal=causal, num_splits=splits,
                                algo="dequant_f16")
        assert_close(out, ref, f"dequant-first {case} splits={splits}")


def _dense_workload(name):
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w)
    return w, inp


@pytest.mark.parametrize("name", ["dense_decode_64k_gqa4", "dense_decode_20k_gqa16"])
def test_dense_decode_workload_full(name):
    w, inp = _dense_workload(name)
    print(f"[dense] {name}", flush=True)
    kp = qkv.qkv_quantize(to_dev(inp["k"], "f16"), "dense")
    vp = qkv.qkv_quantize(to_dev(inp["v"], "f16"), "dense")
    out = qkv.qsdpa_decode(to_dev(inp["q"], "f16"), kp, vp, w.L, w.scale)
    ref = _dense_ref(inp["q"], inp["k"], inp["v"], "f16", w.scale)
    assert_close(out, ref, name, report=True)


def test_dequantize_first_prefill_workload_all_rows():
    w = W.WORKLOADS["q8_0_prefill_512"]
    print("[dequant-first] q8_0_prefill_512", flush=True)
    inp = W.make_inputs(w)
    kp = qkv.qkv_quantize(to_dev(inp["k"], w.dtype), w.mode, w.bits, w.group_size)
    vp = qkv.qkv_quantize(to_dev(inp["v"], w.dtype), w.mode, w.bits, w.group_size)
    kr = oracle_pack(inp["k"], w.dtype, w.mode, w.bits, w.group_size)
    vr = oracle_pack(inp["v"], w.dtype, w.mode, w.bits, w.group_size)
    out = qkv.qsdpa_prefill(to_dev(inp["q"], w.dtype), kp, vp, w.L, w.scale, causal=True,
                            algo="dequant_f16")
    ref = oracle_attention(inp["q"], w.dtype, kr, vr, w.L, w.mode, w.bits, w.group_size, w.scale,
                           causal=True)
    assert_close(out, ref, "dequant-first prefill all 512 rows", report=True)
