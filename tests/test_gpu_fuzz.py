"""Seeded random shapes against the oracle: formats, query dtypes, head sizes,
GQA factors, lengths with ragged tails, query counts, causal and additive
masks, and split counts, so every attention kernel (the narrow and 16-head
decodes, the tiled prefill, the generic kernel) and both split merges see
shapes no hand-written case pins.  Draws are fixed by the case index."""
import numpy as np
import pytest
import torch

import quantized_kv_cache_amd as qkv
from quantized_kv_cache_amd import _lib
from tests._cases import W, assert_close, assert_pack_equal, oracle_attention, oracle_pack, pack_numpy, to_dev

pytestmark = pytest.mark.gpu

FORMATS = [("affine", 4, 32), ("affine", 4, 64), ("affine", 4, 128), ("affine", 8, 32),
           ("affine", 8, 64), ("affine", 8, 128), ("q8_0", 8, 32)]


def draw(i):
    rng = np.random.default_rng(7000 + i)
    mode, bits, gs = FORMATS[rng.integers(len(FORMATS))]
    D = int(rng.choice([64, 128, 256]))
    if D % gs:
        D = 128
    dtype = str(rng.choice(["f16", "f16", "f16", "bf16", "f32"]))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    Hk = int(rng.integers(1, 4))
    B = int(rng.integers(1, 3))
    Lq = int(rng.choice([1, 1, 1, 2, 7, 33]))
    L = int(rng.integers(max(Lq, 1), 2500))
    mask = str(rng.choice(["none", "none", "causal", "additive"])) if Lq > 1 else \
        str(rng.choice(["none", "none", "additive"]))
    splits = int(rng.choice([0, 0, 1, 2, 5, 33]))
    return mode, bits, gs, D, dtype, G, Hk, B, Lq, L, mask, splits


@pytest.mark.parametrize("i", range(96))
def test_attention_fuzz(i):
    mode, bits, gs, D, dtype, G, Hk, B, Lq, L, mask, splits = case = draw(i)
    print(f"[fuzz {i}] {case}", flush=True)
    Hq = G * Hk
    s = 9000 + 17 * i
    q = W.random_case(s, (B, Hq, Lq, D), "normal", dtype)
    k = W.random_case(s + 1, (B, Hk, L, D), "normal", dtype)
    v = W.random_case(s + 2, (B, Hk, L, D), "normal", dtype)
    kp = qkv.qkv_quantize(to_dev(k, dtype), mode, bits, gs)
    vp = qkv.qkv_quantize(to_dev(v, dtype), mode, bits, gs)
    kr, vr = oracle_pack(k, dtype, mode, bits, gs), oracle_pack(v, dtype, mode, bits, gs)
    assert_pack_equal(pack_numpy(kp), kr)
    assert_pack_equal(pack_numpy(vp), vr)
    scale = float(1.0 / np.sqrt(D))
    m = None
    if mask == "additive":
        rng = np.random.default_rng(s + 3)
        m = (rng.standard_normal((B, Hq, Lq, L)) * 2.0).astype(np.float32)
        m[rng.random((B, Hq, Lq, L)) < 0.1] = -np.inf
        m[..., 0] = 0.0                                   # every row sees key 0
    qd = to_dev(q, dtype)
    md = None if m is None else torch.from_numpy(m).cuda()
    try:
        if Lq == 1:
            out = qkv.qsdpa_decode(qd, kp, vp, L, scale, mask=md, num_splits=splits)
        else:
            out = qkv.qsdpa_prefill(qd, kp, vp, L, scale, causal=(mask == "causal"), mask=md,
                                    num_splits=splits)
    except _lib.QKVError as e:
        assert e.status == _lib.QKV_EUNSUPPORTED, str(e)
        pytest.skip(f"unsupported combination: {e}")
    ref = oracle_attention(q, dtype, kr, vr, L, mode, bits, gs, scale, mask=m, causal=(mask == "causal"))
    assert_close(out, ref, f"fuzz {i} {case}")
