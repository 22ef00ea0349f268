"""Attention at the largest cache the matrix-core kernels address (a kv head's
rows span just under 2^31 bytes, the limit of their 32-bit offsets) and just
past it (where the plan falls back to the generic kernel and its 64-bit row
offsets).

A check that still discriminates at these sizes without running the oracle
over millions of keys: every key row holds one "cold" row whose score is
about -45 below the "hot" rows' for every head, and a few hot rows are written
by qkv_update_append at offsets spread over the span, the last ones at the
span's end.  Each cold key then weighs below e^-40 next to a hot one, so the
output is, to far inside the tolerance, the attention over the hot rows alone
-- which the oracle computes from the hot rows' host values.  A kernel that
misaddresses rows near 2^31 bytes, drops a split or mis-merges reads the wrong
values for some hot key and fails.  The hot rows of the packs are checked bit
for bit against the oracle's quantization of the same values.
"""
import math

import numpy as np
import pytest
import torch

import quantized_kv_cache_amd as qkv
from tests._cases import (assert_close, assert_pack_equal, oracle_attention, oracle_pack,
                          pack_numpy)

pytestmark = pytest.mark.gpu


def _hot_positions(L: int, rng: np.random.Generator) -> list:
    fixed = [0, 1, L // 3, L // 2, L - 4096, L - 65, L - 2, L - 1]
    extra = rng.choice(np.arange(2, L - 2), size=8, replace=False).tolist()
    return sorted(set(int(j) for j in fixed + extra))


@pytest.mark.parametrize("mode,bits,gs,D,G,Lq,L,kernel", [
    # 8-bit codes, D = 128: 128 bytes per row, 2^24 - 1 rows = 2^31 - 128 bytes
    ("affine", 8, 64, 128, 4, 1, (1 << 24) - 1, "attn_decode_narrow"),
    # one more 64-key tile than 2^31 bytes: the generic kernel
    ("affine", 8, 64, 128, 4, 1, (1 << 24) + 64, "attn_generic_kernel"),
    # Q8_0, D = 256: 256 bytes per row, 2^23 - 1 rows
    ("q8_0", 8, 32, 256, 16, 1, (1 << 23) - 1, "attn_matrix_decode"),
    ("q8_0", 8, 32, 256, 16, 4, (1 << 23) - 1, "attn_matrix_prefill"),
])
def test_hot_keys_at_the_addressing_limit(mode, bits, gs, D, G, Lq, L, kernel):
    print(f"[max-size] {mode} {bits} D={D} G={G} Lq={Lq} L={L} ({kernel})", flush=True)
    seed = (L * 31 + D * 7 + G + Lq) % 100003
    rng = np.random.default_rng(seed)
    B, Hk, Hq = 1, 1, G
    scale = 1.0 / math.sqrt(D)
    # queries: a common direction u plus a small per-head part, so that one
    # cold row (-2 u) is far below every head's hot rows (+2 u + noise)
    u = rng.standard_normal(D).astype(np.float32)
    q = (u[None, None, None, :] + 0.1 * rng.standard_normal((B, Hq, Lq, D))).astype(np.float16)
    cold = (-2.0 * u).astype(np.float16)[None, None, None, :]
    hot = _hot_positions(L, rng)
    k_hot = (2.0 * u[None, :] + 0.5 * rng.standard_normal((len(hot), D))).astype(np.float16)
    v_hot = rng.standard_normal((len(hot), D)).astype(np.float16)

    dev = torch.device("cuda")
    gen = torch.Generator(device=dev).manual_seed(seed)
    k_src = torch.from_numpy(cold).to(dev).expand(B, Hk, L, D)         # one row, stride 0 along L
    v_src = torch.randn((B, Hk, L, D), generator=gen, device=dev, dtype=torch.float16)
    kp = qkv.qkv_quantize(k_src, mode, bits, gs)
    vp = qkv.qkv_quantize(v_src, mode, bits, gs)
    del v_src
    for n, j in enumerate(hot):
        qkv.qkv_update_append(kp, vp, torch.from_numpy(k_hot[n][None, None, None, :]).to(dev),
                              torch.from_numpy(v_hot[n][None, None, None, :]).to(dev), j)
    torch.cuda.synchronize()

    # the hot rows of the packs, against the oracle's quantization of their values
    idx = torch.tensor(hot, device=dev)
    def rows(p):
        sel = dict(codes=p.codes[:, :, idx], scales=p.scales[:, :, idx],
                   biases=None if p.biases is None else p.biases[:, :, idx])
        return pack_numpy(qkv.Pack(p.mode, p.bits, p.group_size, p.D, **sel))
    kr = oracle_pack(k_hot[None, None], "f16", mode, bits, gs)
    vr = oracle_pack(v_hot[None, None], "f16", mode, bits, gs)
    assert_pack_equal(rows(kp), kr)
    assert_pack_equal(rows(vp), vr)
    # a cold row too
    kc = oracle_pack(cold, "f16", mode, bits, gs)
    one = torch.tensor([L // 4], device=dev)
    assert_pack_equal(pack_numpy(qkv.Pack(kp.mode, kp.bits, kp.group_size, kp.D, kp.codes[:, :, one],
                                          kp.scales[:, :, one],
                                          None if kp.biases is None else kp.biases[:, :, one])), kc)

    qd = torch.from_numpy(q).to(dev)
    assert qkv.qsdpa_plan(qd, kp, L)["kernel"] == kernel
    if Lq == 1:
        out = qkv.qsdpa_decode(qd, kp, vp, L, scale)
    else:
        out = qkv.qsdpa_prefill(qd, kp, vp, L, scale)
    ref = oracle_attention(q, "f16", kr, vr, len(hot), mode, bits, gs, scale)
    # the cold keys' share of the softmax, bounded from the oracle's own scores
    assert_close(out, ref, f"hot keys at L={L} ({kernel})", report=True)
