"""GPU parity of qkv_quantize and qkv_update_append: packed codes, scales and
biases must equal the oracle's bit for bit."""
import zlib

import numpy as np
import pytest
import torch

import quantized_kv_cache_amd as qkv
from tests._cases import (W, assert_pack_equal, oracle_pack, pack_numpy, to_dev)

pytestmark = pytest.mark.gpu

FORMATS = [("affine", 4, 32), ("affine", 4, 64), ("affine", 4, 128), ("affine", 8, 32),
           ("affine", 8, 64), ("affine", 8, 128), ("q8_0", 8, 32)]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("mode,bits,gs", FORMATS)
@pytest.mark.parametrize("D", [64, 128, 256])
def test_quantize_fuzz_bitexact(dtype, mode, bits, gs, D):
    if mode == "affine" and D % gs:
        pytest.skip("group does not divide D")
    seed = zlib.crc32(f"{dtype}{mode}{bits}{gs}{D}".encode()) % 10000
    x = W.random_case(seed, (2, 3, 37, D), "normal" if seed % 2 else "uniform", dtype)
    x[0, 0, 3] = x[0, 0, 3, 0]                  # a constant row (eps scale)
    x[1, 2, 5, :32] = 0                         # a zero block
    pk = qkv.qkv_quantize(to_dev(x, dtype), mode, bits, gs)
    assert_pack_equal(pack_numpy(pk), oracle_pack(x, dtype, mode, bits, gs))


@pytest.mark.parametrize("name", [n for n, w in W.WORKLOADS.items() if w.mode != "dense"])
def test_quantize_workload_bitexact(name):
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w)
    print(f"[quantize] {name} K,V {inp['k'].shape} {w.dtype}", flush=True)
    for t in ("k", "v"):
        pk = qkv.qkv_quantize(to_dev(inp[t], w.dtype), w.mode, w.bits, w.group_size)
        assert_pack_equal(pack_numpy(pk), oracle_pack(inp[t], w.dtype, w.mode, w.bits,
                                                      w.group_size))
        del pk
        torch.cuda.empty_cache()


@pytest.mark.parametrize("mode,bits,gs", [("affine", 4, 64), ("affine", 8, 64), ("q8_0", 8, 32)])
def test_quantize_strided_source_and_pack(mode, bits, gs):
    """A non-contiguous source (every other token) into a pack laid out as
    [B, L_cap, H] rows viewed as [B, H, L_cap]."""
    B, H, L, D = 2, 4, 24, 128
    full = W.random_case(9, (B, H, 2 * L, D), "normal", "f16")
    xs = full[:, :, ::2]
    xt = to_dev(full, "f16")[:, :, ::2]
    dense = qkv.empty_pack(B, L, H, D, mode, bits, gs, torch.float16)   # [B, L, H, .]
    perm = qkv.Pack(mode, bits, gs, D, dense.codes.transpose(1, 2), dense.scales.transpose(1, 2),
                    None if dense.biases is None else dense.biases.transpose(1, 2))
    qkv.qkv_quantize(xt, out=perm)
    assert_pack_equal(pack_numpy(perm), oracle_pack(np.ascontiguousarray(xs), "f16", mode, bits, gs))


@pytest.mark.parametrize("mode,bits,gs", [("affine", 4, 64), ("affine", 8, 32), ("q8_0", 8, 32)])
@pytest.mark.parametrize("T,offset", [(1, 0), (1, 40), (3, 17), (48, 0)])
def test_append_bitexact_untouched_rows(mode, bits, gs, T, offset):
    B, H, Lcap, D = 2, 3, 48, 128
    base = W.random_case(21, (B, H, Lcap, D), "normal", "f16")
    new = W.random_case(22, (2, B, H, T, D), "normal", "f16")
    kc = qkv.qkv_quantize(to_dev(base, "f16"), mode, bits, gs)
    vc = qkv.qkv_quantize(to_dev(base[:, :, ::-1].copy(), "f16"), mode, bits, gs)
    k_before, v_before = pack_numpy(kc), pack_numpy(vc)
    qkv.qkv_update_append(kc, vc, to_dev(new[0], "f16"), to_dev(new[1], "f16"), offset)
    kref = oracle_pack(new[0], "f16", mode, bits, gs)
    vref = oracle_pack(new[1], "f16", mode, bits, gs)
    rows = slice(offset, offset + T)
    k_after, v_after = pack_numpy(kc), pack_numpy(vc)
    assert_pack_equal({k: None if a is None else a[:, :, rows] for k, a in k_after.items()}, kref)
    assert_pack_equal({k: None if a is None else a[:, :, rows] for k, a in v_after.items()}, vref)
    others = np.r_[0:offset, offset + T:Lcap]
    assert_pack_equal(k_after, k_before, rows=others)
    assert_pack_equal(v_after, v_before, rows=others)


def test_append_workload_steps():
    """The batched append workload: a few steps of appending one token per
    sequence at rows 16384 + t (B=8, Hk=8, D=128, 8-bit, group 64)."""
    w = W.WORKLOADS["append_decode_b8_8bit"]
    B, Hk, D = w.B, w.Hk, w.D
    kc = qkv.empty_pack(B, Hk, w.cap, D, w.mode, w.bits, w.group_size, torch.float16)
    vc = qkv.empty_pack(B, Hk, w.cap, D, w.mode, w.bits, w.group_size, torch.float16)
    rng = np.random.default_rng(w.seed)
    for t in range(4):
        s = W.append_step_inputs(w, rng)
        qkv.qkv_update_append(kc, vc, to_dev(s["k_new"], "f16"), to_dev(s["v_new"], "f16"),
                              w.L + t)
        got_k = {k: None if a is None else a[:, :, w.L + t:w.L + t + 1]
                 for k, a in pack_numpy(kc).items()}
        got_v = {k: None if a is None else a[:, :, w.L + t:w.L + t + 1]
                 for k, a in pack_numpy(vc).items()}
        assert_pack_equal(got_k, oracle_pack(s["k_new"], "f16", w.mode, w.bits, w.group_size))
        assert_pack_equal(got_v, oracle_pack(s["v_new"], "f16", w.mode, w.bits, w.group_size))


def test_quantize_rejects_bad_arguments():
    x = torch.zeros((1, 1, 8, 128), dtype=torch.float16, device="cuda")
    pk = qkv.empty_pack(1, 1, 4, 128)
    with pytest.raises(qkv.QKVError, match="QKV_EINVAL"):
        qkv.qkv_quantize(x, out=pk)           # L=8 > L_cap=4
    before = pack_numpy(pk)
    with pytest.raises(qkv.QKVError):
        qkv.qkv_update_append(pk, pk, x[:, :, :2], x[:, :, :2], 3)   # rows 3..5 > cap
    assert_pack_equal(pack_numpy(pk), before)


# exact ties on the GPU: rows whose quotients are exactly k + 1/2 (the
# hand-derived fixtures under tests/golden/), repeated over rows, heads and
# both halves of a D = 128 row, so every lane position of the kernel meets
# them; codes, scales and biases must be the fixtures' own values
def _unpack_codes(words: np.ndarray, bits: int, D: int) -> np.ndarray:
    w = np.ascontiguousarray(words).view(np.uint32).astype(np.uint64)
    per = 32 // bits
    j = np.arange(D)
    return ((w[..., j // per] >> ((j % per) * bits).astype(np.uint64)) & ((1 << bits) - 1)).astype(np.int64)


@pytest.mark.parametrize("name,D", [("affine_ties_4bit_g32.txt", 64), ("affine_ties_4bit_g32.txt", 128),
                                    ("affine_ties_8bit_g32.txt", 64), ("affine_ties_8bit_g32.txt", 128),
                                    ("q8_0_ties.txt", 64), ("q8_0_ties.txt", 256)])
def test_quantize_exact_ties_match_golden(name, D):
    from tests import _golden
    g = _golden.load(name)
    row = np.asarray(g["x"], np.float16)
    assert np.array_equal(row.astype(np.float64), np.asarray(g["x"], np.float64))
    reps = D // row.size
    x = np.tile(row, (2, 3, 37, reps))                        # [B, H, L, D]
    xd = to_dev(x, "f16")
    if name.startswith("q8_0"):
        pk = pack_numpy(qkv.qkv_quantize(xd, "q8_0", 8, 32))
        codes = pk["codes"].astype(np.int64)
        assert np.array_equal(codes, np.broadcast_to(np.tile(np.asarray(g["codes"]), reps), codes.shape))
        d = pk["scales"].view(np.float16).astype(np.float64)
        assert np.array_equal(d, np.broadcast_to(np.tile(np.asarray(g["d"], np.float64), reps), d.shape))
    else:
        bits = g["bits"]
        pk = pack_numpy(qkv.qkv_quantize(xd, "affine", bits, 32))
        codes = _unpack_codes(pk["codes"], bits, D)
        assert np.array_equal(codes, np.broadcast_to(np.tile(np.asarray(g["codes_unpacked"]), reps), codes.shape))
        for key in ("scales", "biases"):
            got = pk[key].astype(np.float64)
            assert np.array_equal(got, np.broadcast_to(np.tile(np.asarray(g[key], np.float64), reps), got.shape)), key


# rows whose rounding decisions are the hard ones: exact k + 1/2 quotients,
# constant rows, and groups of fp16 subnormal steps (values o + k 2^-24 with
# a range of R steps).  With R steps the scale R/15 (R/255) is stored as an
# fp16 multiple of 2^-24, so for R below a few hundred its rounding moves the
# top quotient well past the last code (R = 36: scale 2 steps, quotient 18);
# the codes must then saturate exactly as the oracle clamps them.
SUBNORMAL_RANGES = (6, 20, 36, 37, 45, 100, 250, 600, 1000)


def _hard_rows(D: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = []
    for num, den in ((1, 16), (7, 128), (3, 64)):
        for bias in (0.0, -2.0):
            k = rng.integers(0, 15, D)
            rows.append(bias + (k + 0.5 * (rng.random(D) < 0.6)) * num / den)
            rows[-1][0], rows[-1][1] = bias, bias + 15 * num / den
    rows.append(np.full(D, 0.3125))
    rows.append(np.full(D, 2.0 ** -24))
    step = 2.0 ** -24
    for R in SUBNORMAL_RANGES:
        for off in (0.0, -R * step, 2.0 ** -14):
            r = off + rng.integers(0, R + 1, D) * step
            r[0::32], r[1::32] = off, off + R * step        # every 32-block spans R steps
            rows.append(r)
    return np.stack(rows).astype(np.float32)


def _top_quotients_f16(x: np.ndarray, bits: int, gs: int) -> np.ndarray:
    """(max - min) / fp16(max(range / (2^bits - 1), fp16(1e-7))) per group,
    in fp32: where this exceeds 2^bits - 1/2 the code has to saturate."""
    g = x.astype(np.float32).reshape(x.shape[0], -1, gs)
    mn, mx = g.min(-1), g.max(-1)
    s = np.maximum((mx - mn) / np.float32(2 ** bits - 1), np.float32(np.float16(1e-7)))
    s = s.astype(np.float16).astype(np.float32)
    return (mx - mn) / s


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("mode,bits,gs", FORMATS)
@pytest.mark.parametrize("D", [64, 256])
def test_quantize_hard_rows_bitexact(dtype, mode, bits, gs, D):
    if mode == "affine" and D % gs:
        pytest.skip("group does not divide D")
    rows = _hard_rows(D, 50 + D + gs)
    x = W.cast(rows, dtype)
    if dtype == "f16" and mode == "affine":
        top = _top_quotients_f16(x.astype(np.float32), bits, gs)
        assert (top > 2 ** bits - 0.5).any(), "no group reaches the saturating codes"
    x = np.broadcast_to(x, (2, 3) + x.shape).copy()          # [B, H, L, D]
    pk = qkv.qkv_quantize(to_dev(x, dtype), mode, bits, gs)
    assert_pack_equal(pack_numpy(pk), oracle_pack(x, dtype, mode, bits, gs))
