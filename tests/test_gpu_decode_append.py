"""Decode with append (qsdpa_decode_append): one step of a decoding loop, the
new K/V token quantized into the cache and the updated cache attended.  The
cache rows must be the bits qkv_update_append writes (so, the oracle's), and
the output must be what qsdpa_decode returns on the updated packs -- the same
kernel with the same plan, so the same bits -- and within the tolerance of
the oracle's attention."""
import dataclasses

import numpy as np
import pytest
import torch

import quantized_kv_cache_amd as qkv
from tests._cases import (assert_close, assert_pack_equal, oracle_attention, oracle_pack, pack_numpy,
                          to_dev, W)

pytestmark = pytest.mark.gpu


def _packs(x, dtype, mode, bits, gs, cap):
    """Packs of capacity cap holding the quantized rows of x [B,H,L0,D]."""
    B, H, L0, D = x.shape
    p = qkv.empty_pack(B, H, cap, D, mode, bits, gs, qkv.torch_dtype(dtype))
    qkv.qkv_quantize(to_dev(x, dtype), out=p)
    return p


def _clone(p):
    return dataclasses.replace(p, codes=p.codes.clone(), scales=p.scales.clone(),
                               biases=None if p.biases is None else p.biases.clone())


CASES = [
    # dtype, mode, bits, gs, B, Hq, Hk, L0, D, splits, steps -- fp16 queries with a
    # GQA factor <= 16 run on the narrow or the 16-row decode (one launch); the
    # others append first
    ("f16", "affine", 8, 64, 2, 8, 4, 1000, 128, 0, 3),      # G = 2
    ("f16", "affine", 4, 64, 1, 16, 4, 4000, 128, 0, 2),     # G = 4
    ("f16", "affine", 4, 32, 1, 4, 4, 70, 64, 0, 3),         # the new row in a wave's first tile
    ("f16", "affine", 8, 32, 2, 6, 2, 2500, 64, 7, 2),       # odd split count, 2 groups
    ("f16", "affine", 4, 128, 3, 12, 3, 777, 128, 3, 2),     # batch 3, G = 4
    ("f16", "q8_0", 8, 32, 1, 8, 2, 513, 128, 0, 3),         # Q8_0
    ("f16", "q8_0", 8, 32, 1, 32, 2, 3000, 256, 0, 2),       # GQA 16: the 16-row decode, one launch
    ("f16", "affine", 4, 64, 1, 16, 2, 1500, 128, 5, 2),     # GQA 8: the folded 16-row decode, 5 splits
    ("f16", "affine", 8, 64, 2, 16, 2, 100, 64, 0, 3),       # GQA 8, the new row in a wave's first tile
    ("f16", "q8_0", 8, 32, 1, 20, 2, 260, 256, 0, 2),        # GQA 10, short cache
    ("f32", "affine", 8, 64, 1, 4, 1, 200, 64, 0, 2),        # fp32: generic kernel after the append
    ("bf16", "affine", 4, 64, 2, 8, 2, 900, 128, 0, 2),      # bf16: generic kernel after the append
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_append_matches_append_then_decode(case):
    dtype, mode, bits, gs, B, Hq, Hk, L0, D, splits, steps = case
    print(f"[decode_append] {case}", flush=True)
    rng = np.random.default_rng(7 + L0)
    cap = L0 + steps
    base_k = W.draw(rng, (B, Hk, L0, D), "normal", dtype)
    base_v = W.draw(rng, (B, Hk, L0, D), "normal", dtype)
    kf, vf = _packs(base_k, dtype, mode, bits, gs, cap), _packs(base_v, dtype, mode, bits, gs, cap)
    ku, vu = _clone(kf), _clone(vf)
    kr = oracle_pack(base_k, dtype, mode, bits, gs)
    vr = oracle_pack(base_v, dtype, mode, bits, gs)
    kr = {n: None if a is None else np.concatenate([a, np.zeros(a.shape[:2] + (steps,) + a.shape[3:], a.dtype)], 2)
          for n, a in kr.items()}
    vr = {n: None if a is None else np.concatenate([a, np.zeros(a.shape[:2] + (steps,) + a.shape[3:], a.dtype)], 2)
          for n, a in vr.items()}
    ws_f, ws_u = qkv.Workspace(), qkv.Workspace()
    scale = 1.0 / np.sqrt(D)
    for t in range(steps):
        k_new = W.draw(rng, (B, Hk, 1, D), "normal", dtype)
        v_new = W.draw(rng, (B, Hk, 1, D), "normal", dtype)
        q = W.draw(rng, (B, Hq, 1, D), "normal", dtype)
        qd = to_dev(q, dtype)
        off = L0 + t
        out_f = qkv.qsdpa_decode_append(qd, kf, vf, to_dev(k_new, dtype), to_dev(v_new, dtype), off, scale,
                                        num_splits=splits, workspace=ws_f)
        qkv.qkv_update_append(ku, vu, to_dev(k_new, dtype), to_dev(v_new, dtype), off)
        out_u = qkv.qsdpa_decode(qd, ku, vu, off + 1, scale, num_splits=splits, workspace=ws_u)
        for ref, new in ((kr, k_new), (vr, v_new)):
            for n, a in oracle_pack(new, dtype, mode, bits, gs).items():
                if a is not None:
                    ref[n][:, :, off] = a[:, :, 0]
        assert_pack_equal(pack_numpy(kf), kr, rows=slice(0, off + 1))
        assert_pack_equal(pack_numpy(vf), vr, rows=slice(0, off + 1))
        assert torch.equal(out_f, out_u), f"step {t}: differs from qkv_update_append + qsdpa_decode"
        ref = oracle_attention(q, dtype, kr, vr, off + 1, mode, bits, gs, scale)
        assert_close(out_f, ref, f"decode_append {case} step {t}")


def test_decode_append_additive_mask():
    """With an additive mask the append runs first and the masked decode
    follows; the result equals the two calls and the oracle."""
    B, Hq, Hk, L0, D = 1, 8, 2, 600, 128
    rng = np.random.default_rng(3)
    base_k = W.draw(rng, (B, Hk, L0, D), "normal", "f16")
    base_v = W.draw(rng, (B, Hk, L0, D), "normal", "f16")
    kf, vf = _packs(base_k, "f16", "affine", 4, 64, L0 + 1), _packs(base_v, "f16", "affine", 4, 64, L0 + 1)
    ku, vu = _clone(kf), _clone(vf)
    k_new = W.draw(rng, (B, Hk, 1, D), "normal", "f16")
    v_new = W.draw(rng, (B, Hk, 1, D), "normal", "f16")
    q = W.draw(rng, (B, Hq, 1, D), "normal", "f16")
    mask = np.where(rng.random((B, Hq, 1, L0 + 1)) < 0.3, -np.inf, rng.normal(size=(B, Hq, 1, L0 + 1)))
    mask[..., -1] = 0.5                               # the new key is visible
    md = torch.from_numpy(mask.astype(np.float32)).cuda()
    qd = to_dev(q, "f16")
    out_f = qkv.qsdpa_decode_append(qd, kf, vf, to_dev(k_new, "f16"), to_dev(v_new, "f16"), L0, 0.1, mask=md)
    qkv.qkv_update_append(ku, vu, to_dev(k_new, "f16"), to_dev(v_new, "f16"), L0)
    out_u = qkv.qsdpa_decode(qd, ku, vu, L0 + 1, 0.1, mask=md)
    assert torch.equal(out_f, out_u)
    kr = oracle_pack(np.concatenate([base_k, k_new], 2), "f16", "affine", 4, 64)
    vr = oracle_pack(np.concatenate([base_v, v_new], 2), "f16", "affine", 4, 64)
    assert_pack_equal(pack_numpy(kf), kr)
    assert_close(out_f, oracle_attention(q, "f16", kr, vr, L0 + 1, "affine", 4, 64, 0.1, mask=mask), "masked")


def test_decode_append_workload_all_steps():
    """The batched append+decode workload at full size through the one-launch
    call, all 64 steps (B=8, Hq=32, Hk=8, D=128, cache 16384 + t, 8-bit, the
    last step filling row 16447): the cache is bit-exact against the oracle's
    rows after the last step, and the attention is checked against the oracle
    at the first steps and the last."""
    w = W.WORKLOADS["append_decode_b8_8bit"]
    print("[decode_append] full size", flush=True)
    inp = W.make_inputs(w)
    rng = inp["rng"]
    kp = qkv.empty_pack(w.B, w.Hk, w.cap, w.D, w.mode, w.bits, w.group_size, torch.float16)
    vp = qkv.empty_pack(w.B, w.Hk, w.cap, w.D, w.mode, w.bits, w.group_size, torch.float16)
    qkv.qkv_quantize(to_dev(inp["k"], "f16"), out=kp)
    qkv.qkv_quantize(to_dev(inp["v"], "f16"), out=vp)
    plan = qkv.qsdpa_plan(to_dev(inp["q"], "f16"), kp, w.cap)
    assert plan["kernel"] == "attn_decode_narrow"
    refs = []
    for src in ("k", "v"):
        pk = oracle_pack(inp[src], "f16", w.mode, w.bits, w.group_size)
        full = {n: np.zeros(a.shape[:2] + (w.cap,) + a.shape[3:], a.dtype) for n, a in pk.items()}
        for n, a in pk.items():
            full[n][:, :, :w.L] = a
        refs.append(full)
    kr, vr = refs
    ws = qkv.Workspace()
    for t in range(w.steps):
        s = W.append_step_inputs(w, rng)
        L = w.L + t + 1
        out = qkv.qsdpa_decode_append(to_dev(s["q"], "f16"), kp, vp, to_dev(s["k_new"], "f16"),
                                      to_dev(s["v_new"], "f16"), w.L + t, w.scale, workspace=ws)
        for ref, new in ((kr, s["k_new"]), (vr, s["v_new"])):
            for n, a in oracle_pack(new, "f16", w.mode, w.bits, w.group_size).items():
                ref[n][:, :, w.L + t] = a[:, :, 0]
        if t in (0, 2, w.steps - 1):
            ref = oracle_attention(s["q"], "f16", kr, vr, L, w.mode, w.bits, w.group_size, w.scale)
            assert_close(out, ref, f"decode_append step {t} (L={L})", report=True)
    assert_pack_equal(pack_numpy(kp), kr)
    assert_pack_equal(pack_numpy(vp), vr)


@pytest.mark.parametrize("mode,bits,gs,Hq", [("affine", 4, 64, 8), ("q8_0", 8, 32, 32)])
def test_decode_append_strided_new_tokens(mode, bits, gs, Hq):
    """The new tokens as a view (one position of a [B, Hk, 5, D] tensor, so
    strides 5 D per head and 5 Hk D per batch): the kernel reads them through
    the strides; cache and output as with a contiguous copy."""
    B, Hk, L0, D = 2, 2, 3000, 128
    rng = np.random.default_rng(11)
    base_k = W.draw(rng, (B, Hk, L0, D), "normal", "f16")
    base_v = W.draw(rng, (B, Hk, L0, D), "normal", "f16")
    kf, vf = _packs(base_k, "f16", mode, bits, gs, L0 + 1), _packs(base_v, "f16", mode, bits, gs, L0 + 1)
    ku, vu = _clone(kf), _clone(vf)
    big_k = W.draw(rng, (B, Hk, 5, D), "normal", "f16")
    big_v = W.draw(rng, (B, Hk, 5, D), "normal", "f16")
    q = W.draw(rng, (B, Hq, 1, D), "normal", "f16")
    qd = to_dev(q, "f16")
    kv, vv = to_dev(big_k, "f16")[:, :, 3:4], to_dev(big_v, "f16")[:, :, 3:4]
    assert not kv.is_contiguous()
    out_f = qkv.qsdpa_decode_append(qd, kf, vf, kv, vv, L0, 0.125)
    qkv.qkv_update_append(ku, vu, kv.contiguous(), vv.contiguous(), L0)
    out_u = qkv.qsdpa_decode(qd, ku, vu, L0 + 1, 0.125)
    assert torch.equal(out_f, out_u)
    for got, want in ((kf, ku), (vf, vu)):
        assert_pack_equal(pack_numpy(got), pack_numpy(want))
