"""The unfused composition (algo="unfused": quantized q K^T into a score
buffer, softmax, quantized P V over key chunks, sum of the chunks; the MLX
fallback of quantized_scaled_dot_product_attention) against the oracle, on
small ragged shapes of every format and query dtype, with masks, and at the
full size of the 64K 4-bit GQA-4 and the Q8_0 GQA-16 decode workloads."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_amd as qkv
from tests._cases import (W, assert_close, assert_pack_equal, oracle_attention, oracle_pack,
                          pack_numpy, to_dev)

pytestmark = pytest.mark.gpu


def _case(seed, dtype, mode, bits, gs, B, Hq, Hk, L, D, dist="normal"):
    q = W.random_case(seed, (B, Hq, 1, D), dist, dtype)
    k = W.random_case(seed + 1, (B, Hk, L, D), dist, dtype)
    v = W.random_case(seed + 2, (B, Hk, L, D), dist, dtype)
    kp = qkv.qkv_quantize(to_dev(k, dtype), mode, bits, gs)
    vp = qkv.qkv_quantize(to_dev(v, dtype), mode, bits, gs)
    return q, kp, vp, oracle_pack(k, dtype, mode, bits, gs), oracle_pack(v, dtype, mode, bits, gs)


CASES = [
    # dtype, mode, bits, gs, B, Hq, Hk, L, D
    ("f16", "affine", 4, 64, 1, 32, 8, 3001, 128),
    ("f16", "affine", 8, 32, 2, 8, 2, 777, 64),
    ("f16", "q8_0", 8, 32, 1, 32, 2, 2500, 256),
    ("f16", "affine", 4, 128, 1, 16, 1, 1300, 256),     # G = 16, 4-bit: 4-byte slices
    ("f16", "affine", 4, 32, 3, 6, 3, 65, 64),
    ("f32", "affine", 8, 64, 1, 4, 1, 256, 64),
    ("bf16", "affine", 4, 64, 2, 12, 4, 999, 128),
    ("bf16", "q8_0", 8, 32, 1, 8, 1, 300, 128),
    ("f16", "affine", 8, 128, 1, 2, 2, 1, 128),          # a single key
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_unfused_small(case):
    dtype, mode, bits, gs, B, Hq, Hk, L, D = case
    q, kp, vp, kr, vr = _case(7 + L, dtype, mode, bits, gs, B, Hq, Hk, L, D)
    qd = to_dev(q, dtype)
    plan = qkv.qsdpa_plan(qd, kp, L, algo="unfused")
    assert plan["algo"] == "unfused" and plan["kernel"] == "unfused_scores_kernel"
    scale = 1.0 / math.sqrt(D)
    ref = oracle_attention(q, dtype, kr, vr, L, mode, bits, gs, scale)
    for _ in range(2):
        out = qkv.qsdpa_decode(qd, kp, vp, L, scale, algo="unfused")
        assert_close(out, ref, f"unfused {case}")


def test_unfused_additive_mask_and_fully_masked_row():
    dtype, mode, bits, gs = "f16", "affine", 4, 64
    B, Hq, Hk, L, D = 2, 8, 2, 700, 128
    q, kp, vp, kr, vr = _case(99, dtype, mode, bits, gs, B, Hq, Hk, L, D)
    rng = np.random.default_rng(12)
    mask = (rng.standard_normal((B, Hq, 1, L)) * 2).astype(np.float32)
    mask[rng.random(mask.shape) < 0.3] = -np.inf
    mask[1, 2, 0, :] = -np.inf
    out = qkv.qsdpa_decode(to_dev(q, dtype), kp, vp, L, 0.125, mask=to_dev(mask, "f32"),
                           algo="unfused")
    ref = oracle_attention(q, dtype, kr, vr, L, mode, bits, gs, 0.125, mask=mask)
    assert_close(out, ref, "unfused masked")
    assert torch.all(out[1, 2] == 0)


def test_unfused_rejects_prefill_and_wide_gqa():
    q, kp, vp, _, _ = _case(5, "f16", "affine", 4, 64, 1, 64, 2, 100, 128)
    with pytest.raises(qkv.QKVError, match="unfused"):
        qkv.qsdpa_decode(to_dev(q, "f16"), kp, vp, 100, 0.1, algo="unfused")
    q2 = W.random_case(6, (1, 8, 4, 128), "normal", "f16")
    kp2 = qkv.qkv_quantize(to_dev(W.random_case(7, (1, 2, 100, 128), "normal", "f16"), "f16"),
                           "affine", 4, 64)
    with pytest.raises(qkv.QKVError, match="unfused"):
        qkv.qsdpa_prefill(to_dev(q2, "f16"), kp2, kp2, 100, 0.1, algo="unfused")


C2_NORMAL = dataclasses.replace(W.WORKLOADS["decode_64k_4bit_gqa4"],
                                name="decode_64k_4bit_gqa4_normal", dist="normal",
                                scale=1.0 / math.sqrt(128.0), seed=33)


@pytest.mark.parametrize("name", ["decode_64k_4bit_gqa4", "decode_64k_4bit_gqa4_normal",
                                  "q8_0_decode_gqa16"])
def test_unfused_workload_full(name):
    w = C2_NORMAL if name == C2_NORMAL.name else W.WORKLOADS[name]
    print(f"[unfused] {name}", flush=True)
    inp = W.make_inputs(w)
    kp = qkv.qkv_quantize(to_dev(inp["k"], w.dtype), w.mode, w.bits, w.group_size)
    vp = qkv.qkv_quantize(to_dev(inp["v"], w.dtype), w.mode, w.bits, w.group_size)
    kr = oracle_pack(inp["k"], w.dtype, w.mode, w.bits, w.group_size)
    vr = oracle_pack(inp["v"], w.dtype, w.mode, w.bits, w.group_size)
    assert_pack_equal(pack_numpy(kp), kr)
    qd = to_dev(inp["q"], w.dtype)
    out = qkv.qsdpa_decode(qd, kp, vp, w.L, w.scale, algo="unfused")
    ref = oracle_attention(inp["q"], w.dtype, kr, vr, w.L, w.mode, w.bits, w.group_size, w.scale)
    assert_close(out, ref, f"unfused {name}", report=True)
    fused = qkv.qsdpa_decode(qd, kp, vp, w.L, w.scale)
    assert_close(fused, ref, f"fused {name}")
