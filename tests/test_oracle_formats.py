"""Pins of the oracle's own scalar-format conversions against independent
library routines (numpy's IEEE binary16, torch's bfloat16), exhaustively
where the space is small."""
import numpy as np
import pytest
import torch


def test_f16_to_f32_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.f32_from_f16_bits(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f32_edge_values():
    rng = np.random.default_rng(7)
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -24,
            2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 * 0.99,
            1e-7, 5.96e-8, 6.1e-5, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, np.inf, -np.inf]
    # every fp16 value and the midpoints between neighbours (ties)
    h = np.arange(0, 0x7c00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2
    rand = rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000)
    allv = np.concatenate([np.array(vals), h, mids, -mids, rand]).astype(np.float32)
    return allv


def test_f32_to_f16_matches_numpy(orc):
    x = _f32_edge_values()
    ours = orc.f16_bits_from_f32(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f32_to_bf16_matches_torch(orc):
    rng = np.random.default_rng(11)
    x = np.concatenate([
        _f32_edge_values()[:30000],
        (rng.standard_normal(20000) * 10.0 ** rng.integers(-38, 38, 20000)).astype(np.float32),
        # exact ties between bfloat16 neighbours
        ((np.arange(1, 5000, dtype=np.uint32) << 16) + 0x8000).view(np.float32),
        ((np.arange(1, 5000, dtype=np.uint32) << 16) + 0x7fff).view(np.float32),
        np.array([1e-40, -3e-41, 3.4e38, -3.39e38], np.float32),
    ]).astype(np.float32)
    x = x[np.isfinite(x)]
    ours = orc.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_to_f32(orc):
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    ours = orc.f32_from_bf16_bits(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


@pytest.mark.parametrize("dt,expect", [("f16", 2.0 ** -23), ("f32", np.float32(1e-7))])
def test_eps_values(orc, dt, expect):
    # eps = T(1e-7): in binary16 1e-7 is the subnormal 2 * 2^-24 = 2^-23
    assert orc.affine_eps(dt) == float(expect)
