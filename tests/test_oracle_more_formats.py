"""Pins of the oracle's wider format set: affine codes of 2, 3, 5 and 6 bits
(the pack factors and bytes per pack of the MLX CUDA page's
quantized_utils.cuh, codes in one least-significant-first bit stream per
row), head size 96, and symmetric 32-blocks of 4 and 5 bits (the reading for
the Q4_0 / Q5_0 caches the llama.cpp page names).  Hand-derived packed rows,
brute force, the half-step error bound, grid-aligned round trips, and an
independent numpy re-derivation (np.packbits with little bit order as the
packer)."""
import numpy as np
import pytest

from quantized_kv_cache_amd import workloads as W
from tests import _golden


def _unpack_stream(codes, bits, D):
    """Codes of each row from its bit stream (numpy's unpackbits, little bit order)."""
    b = np.unpackbits(np.ascontiguousarray(codes).view(np.uint8), axis=-1, bitorder="little")
    b = b.reshape(codes.shape[:-1] + (D, bits)).astype(np.int64)
    return (b << np.arange(bits)).sum(-1)


def _pack_stream(c, bits):
    """Rows of codes (non-negative, < 2^bits) -> uint32 words of their bit streams."""
    c = np.asarray(c, np.int64)
    b = ((c[..., None] >> np.arange(bits)) & 1).astype(np.uint8)
    by = np.packbits(b.reshape(c.shape[:-1] + (-1,)), axis=-1, bitorder="little")
    return np.ascontiguousarray(by).view(np.uint32)


@pytest.mark.parametrize("name", ["affine_pack_2bit_g32.txt", "affine_pack_3bit_g32.txt",
                                  "affine_pack_5bit_g32.txt", "affine_pack_6bit_g32.txt"])
def test_golden_stream_rows(orc, name):
    g = _golden.load(name)
    x = W.cast(np.asarray(g["x"], np.float32), "f16")[None, :]
    codes, s, b = orc.quantize_affine(x, "f16", g["bits"], g["group_size"])
    assert [int(w) for w in codes[0]] == g["codes"]
    sc = g["scales"] if isinstance(g["scales"], list) else [g["scales"]]
    bi = g["biases"] if isinstance(g["biases"], list) else [g["biases"]]
    assert orc.to_f32(s, "f16")[0].astype(np.float64).tolist() == sc
    assert orc.to_f32(b, "f16")[0].astype(np.float64).tolist() == bi
    assert np.array_equal(orc.dequant_affine(codes, s, b, "f16", g["bits"], g["group_size"]),
                          x.astype(np.float32))


@pytest.mark.parametrize("name", ["qsym_4bit_block.txt", "qsym_5bit_block.txt"])
def test_golden_symmetric_blocks(orc, name):
    g = _golden.load(name)
    x = W.cast(np.asarray(g["x"], np.float32), "f16")[None, :]
    codes, d = orc.quantize_qsym(x, "f16", g["bits"])
    assert [int(w) for w in codes[0]] == g["codes"]
    assert int(d[0, 0]) == g["d_bits"]
    assert np.array_equal(orc.dequant_qsym(codes, d, g["bits"]), x.astype(np.float32))


AFF = [(2, 32, 256, "f16", "normal"), (3, 64, 128, "f16", "uniform"), (3, 32, 96, "f32", "normal"),
       (5, 32, 96, "f16", "normal"), (5, 128, 256, "bf16", "uniform"), (6, 64, 128, "f16", "normal"),
       (6, 32, 64, "f32", "uniform"), (4, 32, 96, "f16", "normal"), (8, 32, 96, "bf16", "normal")]


@pytest.mark.parametrize("bits,gs,D,dt,dist", AFF)
def test_affine_stream_nearest_bounded_and_rederived(orc, bits, gs, D, dt, dist):
    x = W.random_case(300 + bits * 7 + D, (5, 13, D), dist, dt)
    codes, s, b = orc.quantize_affine(x, dt, bits, gs)
    n = (1 << bits) - 1
    c = _unpack_stream(codes, bits, D)
    assert c.min() >= 0 and c.max() <= n
    xf = orc.to_f32(x, dt).astype(np.float64).reshape(-1, D // gs, gs)
    sf = orc.to_f32(s, dt).astype(np.float64).reshape(-1, D // gs, 1)
    bf = orc.to_f32(b, dt).astype(np.float64).reshape(-1, D // gs, 1)
    cg = c.reshape(xf.shape)
    grid = np.arange(n + 1, dtype=np.float64)
    err_all = np.abs(xf[..., None] - (sf[..., None] * grid + bf[..., None]))
    mine = np.take_along_axis(err_all, cg[..., None], axis=-1)[..., 0]
    assert np.all(mine <= err_all.min(-1) + 1e-5 * sf)
    xh = orc.dequant_affine(codes, s, b, dt, bits, gs).astype(np.float64).reshape(xf.shape)
    ulp = np.spacing(np.abs(xf).astype(np.float32) + np.abs(bf).astype(np.float32)).astype(np.float64)
    short = n * np.maximum(0.0, (xf.max(-1, keepdims=True) - xf.min(-1, keepdims=True)) / n - sf)
    assert np.all(np.abs(xf - xh) <= np.maximum(sf / 2, short) + 2 * ulp)
    # independent re-derivation: numpy fp32 arithmetic, numpy bit packing
    from tests.test_oracle_quant import _np_affine
    c_np, s_np, b_np = _np_affine(x.reshape(-1, D), dt, bits, gs)
    assert np.array_equal(c.reshape(-1, D), c_np)
    assert np.array_equal(codes.reshape(-1, D * bits // 32), _pack_stream(c_np, bits))
    assert np.array_equal(orc.to_f32(s, dt).reshape(-1, D // gs), s_np)


@pytest.mark.parametrize("bits", [2, 3, 5, 6])
def test_affine_stream_grid_aligned_lossless(orc, bits):
    rng = np.random.default_rng(bits)
    rows, D, gs, n = 20, 128, 32, (1 << bits) - 1
    c = rng.integers(0, n + 1, (rows, D // gs, gs))
    c[..., 0], c[..., 1] = 0, n
    k = rng.integers(-64, 65, (rows, D // gs, 1))
    x = ((k + c) / 16.0).reshape(rows, D).astype(np.float16)
    codes, s, b = orc.quantize_affine(x, "f16", bits, gs)
    assert np.array_equal(_unpack_stream(codes, bits, D).reshape(c.shape), c)
    assert np.array_equal(orc.dequant_affine(codes, s, b, "f16", bits, gs), x.astype(np.float32))


def _np_qsym(x, dt, bits):
    from tests.test_oracle_quant import _np_widen
    xf = _np_widen(x, dt)
    D = xf.shape[-1]
    qmax = np.float32((1 << (bits - 1)) - 1)
    g = xf.reshape(-1, D // 32, 32)
    d = (np.abs(g).max(-1, keepdims=True) / qmax).astype(np.float16).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.clip(np.rint(g / d), -qmax, qmax)
    c = np.where(d == 0, np.float32(0), c).astype(np.int64)
    return c.reshape(xf.shape), d[..., 0].reshape(xf.shape[:-1] + (D // 32,))


@pytest.mark.parametrize("bits,D,dt,dist", [(4, 128, "f16", "normal"), (5, 96, "f16", "uniform"),
                                            (4, 256, "bf16", "normal"), (5, 64, "f32", "normal")])
def test_symmetric_blocks(orc, bits, D, dt, dist):
    x = W.random_case(400 + bits + D, (4, 11, D), dist, dt)
    x[0, 0, :32] = 0                                       # an all-zero block
    codes, d = orc.quantize_qsym(x, dt, bits)
    qmax = (1 << (bits - 1)) - 1
    u = _unpack_stream(codes, bits, D)
    c = np.where(u >= (1 << (bits - 1)), u - (1 << bits), u)          # two's complement
    assert c.min() >= -qmax and c.max() <= qmax
    c_np, d_np = _np_qsym(x, dt, bits)
    assert np.array_equal(c.reshape(c_np.shape), c_np)
    assert np.array_equal(orc.to_f32(d, "f16").reshape(d_np.shape), d_np)
    assert np.array_equal(codes.reshape(-1, D * bits // 32),
                          _pack_stream(c_np.reshape(-1, D) & ((1 << bits) - 1), bits))
    xf = orc.to_f32(x, dt).astype(np.float64).reshape(-1, D // 32, 32)
    df = d_np.astype(np.float64).reshape(-1, D // 32, 1)
    cg = c.reshape(xf.shape)
    assert np.all(cg[0, 0] == 0) and df[0, 0, 0] == 0
    nz = df[..., 0] > 0
    ia = np.abs(xf).argmax(-1)[..., None]
    assert np.all(np.abs(np.take_along_axis(cg, ia, -1)[..., 0][nz]) == qmax)
    xh = orc.dequant_qsym(codes, d, bits).astype(np.float64).reshape(xf.shape)
    assert np.all(np.abs(xf - xh) <= df / 2 + 2 * np.spacing(np.abs(xf).astype(np.float32)))
