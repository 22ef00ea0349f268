"""Attention calls captured in a HIP graph (torch.cuda.CUDAGraph on ROCm) and
replayed: the decode with the in-kernel split merge (its merge tickets must
be back at zero after every replay), the 16-row decode followed by the split
merge kernel, the VALU decode followed by its merge kernel, the causal prefill, qsdpa_decode_static (the entry point for
callers that cannot allocate) and qsdpa_decode_append (a decoding step).  Between replays the captured query
tensor is rewritten and the same call runs eagerly on the same workspace;
every replay must equal the eager call bit for bit, and the first of them
the oracle within the attention tolerance."""
import numpy as np
import pytest
import torch

import quantized_kv_cache_amd as qkv
from tests._cases import assert_close, oracle_attention, oracle_pack, to_dev, W

pytestmark = pytest.mark.gpu

CASES = {
    # name: (B, Hq, Hk, Lq, L, D, mode, bits, gs, causal)
    "narrow_fused_merge": (1, 16, 4, 1, 9000, 128, "affine", 4, 64, False),
    "sixteen_row_merge_kernel": (1, 32, 2, 1, 6000, 256, "q8_0", 8, 32, False),
    "prefill_causal": (1, 8, 2, 40, 3000, 128, "q8_0", 8, 32, True),
    "generic_merge_kernel": (1, 4, 1, 1, 6000, 64, "affine", 8, 64, False),
}
ALGO = {"generic_merge_kernel": "generic"}      # the VALU decode and its split merge kernel


def _inputs(seed, B, Hq, Hk, Lq, L, D, mode, bits, gs):
    k = W.random_case(seed + 1, (B, Hk, L, D), "normal", "f16")
    v = W.random_case(seed + 2, (B, Hk, L, D), "normal", "f16")
    kp = qkv.qkv_quantize(to_dev(k, "f16"), mode, bits, gs)
    vp = qkv.qkv_quantize(to_dev(v, "f16"), mode, bits, gs)
    qs = [W.random_case(seed + 10 + r, (B, Hq, Lq, D), "normal", "f16") for r in range(2)]
    return k, v, kp, vp, qs


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_equal_eager_calls(name):
    B, Hq, Hk, Lq, L, D, mode, bits, gs, causal = CASES[name]
    scale = 1.0 / np.sqrt(D)
    k, v, kp, vp, qs = _inputs(71, B, Hq, Hk, Lq, L, D, mode, bits, gs)
    print(f"[graph] {name}", flush=True)
    s = torch.cuda.Stream()
    ws = qkv.Workspace()
    with torch.cuda.stream(s):
        q = to_dev(qs[0], "f16")
        out = torch.empty_like(q)
        call = qkv.PreparedAttention(q, kp, vp, L, scale, out, causal=causal, workspace=ws,
                                     algo=ALGO.get(name, "auto"))
        call()
        call()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for rep in range(4):
        qn = qs[rep % 2]
        q.copy_(to_dev(qn, "f16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        with torch.cuda.stream(s):
            call()                      # the same launch, eagerly, on the same workspace
        s.synchronize()
        assert torch.equal(got, out), f"{name}: replay {rep} differs from the eager call"
        if rep < 2:
            ref = oracle_attention(qn, "f16", oracle_pack(k, "f16", mode, bits, gs),
                                   oracle_pack(v, "f16", mode, bits, gs), L, mode, bits, gs,
                                   scale, causal=causal)
            assert_close(got, ref, f"{name} replay {rep}")
    plan = qkv.qsdpa_plan(q, kp, L, algo=ALGO.get(name, "auto"))
    assert plan["num_splits"] > 1, plan           # the split states and merge are exercised


def test_graph_replays_of_the_static_decode():
    B, Hq, Hk, Lq, L, D, mode, bits, gs, _ = CASES["narrow_fused_merge"]
    scale = 1.0 / np.sqrt(D)
    k, v, kp, vp, qs = _inputs(83, B, Hq, Hk, Lq, L, D, mode, bits, gs)
    print("[graph] static decode", flush=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q = to_dev(qs[0], "f16")
        out = torch.empty_like(q)
        qkv.qsdpa_decode_static(q, kp, vp, L, scale, out=out)   # first call on the device: set-up
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        qkv.qsdpa_decode_static(q, kp, vp, L, scale, out=out)
    for rep in range(4):
        q.copy_(to_dev(qs[rep % 2], "f16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        with torch.cuda.stream(s):
            qkv.qsdpa_decode_static(q, kp, vp, L, scale, out=out)
        s.synchronize()
        assert torch.equal(got, out), f"static decode: replay {rep} differs from the eager call"
        want = qkv.qsdpa_decode(q, kp, vp, L, scale)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"static decode: replay {rep} differs from qsdpa_decode"


def test_graph_replays_of_the_decode_with_append():
    """qsdpa_decode_append captured (one launch on the narrow decode: the new
    row quantized in the kernel, the split merge in the kernel): between
    replays the captured new token and query are rewritten; every replay
    writes the cache row qkv_update_append writes and returns the eager
    decode's output on the updated cache."""
    B, Hq, Hk, L0, D = 2, 8, 4, 5000, 128
    mode, bits, gs = "affine", 8, 64
    scale = 1.0 / np.sqrt(D)
    print("[graph] decode with append", flush=True)
    rng = np.random.default_rng(97)
    base_k = W.draw(rng, (B, Hk, L0, D), "normal", "f16")
    base_v = W.draw(rng, (B, Hk, L0, D), "normal", "f16")
    kp = qkv.empty_pack(B, Hk, L0 + 1, D, mode, bits, gs, torch.float16)
    vp = qkv.empty_pack(B, Hk, L0 + 1, D, mode, bits, gs, torch.float16)
    qkv.qkv_quantize(to_dev(base_k, "f16"), out=kp)
    qkv.qkv_quantize(to_dev(base_v, "f16"), out=vp)
    steps = [{n: W.draw(rng, shp, "normal", "f16") for n, shp in
              (("q", (B, Hq, 1, D)), ("k", (B, Hk, 1, D)), ("v", (B, Hk, 1, D)))} for _ in range(2)]
    s = torch.cuda.Stream()
    ws = qkv.Workspace()
    with torch.cuda.stream(s):
        q = to_dev(steps[0]["q"], "f16")
        kn = to_dev(steps[0]["k"], "f16")
        vn = to_dev(steps[0]["v"], "f16")
        out = torch.empty_like(q)
        call = qkv.PreparedDecodeAppend(q, kp, vp, kn, vn, L0, scale, out, workspace=ws)
        call()
        call()
    s.synchronize()
    assert qkv.qsdpa_plan(q, kp, L0 + 1)["kernel"] == "attn_decode_narrow"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for rep in range(4):
        st = steps[rep % 2]
        q.copy_(to_dev(st["q"], "f16"))
        kn.copy_(to_dev(st["k"], "f16"))
        vn.copy_(to_dev(st["v"], "f16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        for p, src in ((kp, st["k"]), (vp, st["v"])):
            ref = oracle_pack(src, "f16", mode, bits, gs)
            assert np.array_equal(p.codes[:, :, L0].cpu().numpy().view(np.uint32), ref["codes"][:, :, 0])
            assert np.array_equal(p.scales[:, :, L0].cpu().numpy().view(np.uint16), ref["scales"][:, :, 0].view(np.uint16))
            assert np.array_equal(p.biases[:, :, L0].cpu().numpy().view(np.uint16), ref["biases"][:, :, 0].view(np.uint16))
        want = qkv.qsdpa_decode(q, kp, vp, L0 + 1, scale)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"decode with append: replay {rep} differs from the eager decode"
        if rep < 2:
            kr = oracle_pack(np.concatenate([base_k, st["k"]], 2), "f16", mode, bits, gs)
            vr = oracle_pack(np.concatenate([base_v, st["v"]], 2), "f16", mode, bits, gs)
            assert_close(got, oracle_attention(st["q"], "f16", kr, vr, L0 + 1, mode, bits, gs, scale),
                         f"decode with append replay {rep}")
