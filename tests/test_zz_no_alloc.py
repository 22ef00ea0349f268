"""qsdpa_decode_static: the decode with the library's static per-GPU
workspace (for callers that cannot allocate), called through the C ABI, must
give what qsdpa_decode gives with a caller's workspace: on two calls in a row,
the second with a smaller input, and on the oracle's tolerance."""
import numpy as np
import pytest
import torch

import quantized_kv_cache_amd as qkv
from tests._cases import assert_close, oracle_attention, oracle_pack, to_dev, W

pytestmark = pytest.mark.gpu


def _case(seed, B, Hq, Hk, L, D, mode, bits, gs):
    q = W.random_case(seed, (B, Hq, 1, D), "normal", "f16")
    k = W.random_case(seed + 1, (B, Hk, L, D), "normal", "f16")
    v = W.random_case(seed + 2, (B, Hk, L, D), "normal", "f16")
    kp = qkv.qkv_quantize(to_dev(k, "f16"), mode, bits, gs)
    vp = qkv.qkv_quantize(to_dev(v, "f16"), mode, bits, gs)
    ref = oracle_attention(q, "f16", oracle_pack(k, "f16", mode, bits, gs),
                           oracle_pack(v, "f16", mode, bits, gs), L, mode, bits, gs, 0.1)
    return to_dev(q, "f16"), kp, vp, ref


@pytest.mark.parametrize("cases", [
    # (B, Hq, Hk, L, D, mode, bits, gs): a large call, then a smaller one
    [(2, 32, 8, 20000, 128, "affine", 4, 64), (1, 8, 2, 3000, 128, "affine", 4, 64)],   # fused merge
    [(1, 32, 2, 12000, 256, "q8_0", 8, 32), (1, 16, 1, 900, 256, "q8_0", 8, 32)],       # merge kernel
])
def test_static_decode_matches_workspace_decode(cases):
    prepared = [_case(50 + i, *c) for i, c in enumerate(cases)]
    print(f"[no-alloc] cases {cases}", flush=True)
    for rep in range(2):
        for (qd, kp, vp, ref), c in zip(prepared, cases):
            L = c[3]
            want = qkv.qsdpa_decode(qd, kp, vp, L, 0.1)
            out = torch.empty_like(qd)
            torch.cuda.synchronize()
            before = torch.cuda.memory_allocated()
            qkv.qsdpa_decode_static(qd, kp, vp, L, 0.1, out=out)
            torch.cuda.synchronize()
            assert torch.cuda.memory_allocated() == before
            plan = qkv.qsdpa_plan(qd, kp, L)
            assert plan["num_splits"] > 1, plan         # the static workspace is used
            assert torch.equal(out, want), f"rep {rep} {c}: differs from qsdpa_decode"
            assert_close(out, ref, f"static decode rep {rep} {c}")


def test_static_decode_rejects_plans_beyond_its_size():
    """A plan whose split states exceed the static workspace is refused with
    EWORKSPACE before anything runs; fewer splits fit and give the same
    result as a caller's workspace."""
    B, Hq, Hk, L, D = 8, 32, 8, 65536, 128
    kp = qkv.empty_pack(B, Hk, L, D, "affine", 8, 64, torch.float16)
    vp = qkv.empty_pack(B, Hk, L, D, "affine", 8, 64, torch.float16)
    kp.scales.fill_(0.01)
    vp.scales.fill_(0.02)
    vp.biases.copy_(torch.linspace(-1, 1, L, device="cuda").view(1, 1, L, 1).expand_as(vp.biases))
    qd = to_dev(W.random_case(61, (B, Hq, 1, D), "normal", "f16"), "f16")
    need = qkv.qsdpa_plan(qd, kp, L, num_splits=64)["workspace_bytes"]
    assert need > qkv._lib.QKV_STATIC_SCRATCH_BYTES
    with pytest.raises(qkv.QKVError, match="static"):
        qkv.qsdpa_decode_static(qd, kp, vp, L, 0.1, num_splits=64)
    for splits in (4, 8):
        assert qkv.qsdpa_plan(qd, kp, L, num_splits=splits)["workspace_bytes"] <= \
            qkv._lib.QKV_STATIC_SCRATCH_BYTES
        out = qkv.qsdpa_decode_static(qd, kp, vp, L, 0.1, num_splits=splits)
        assert torch.equal(out, qkv.qsdpa_decode(qd, kp, vp, L, 0.1, num_splits=splits))
