"""Pins of the oracle's number codecs against library casts (torch, numpy)."""
import numpy as np
import pytest
import torch


def test_bf16_decode_all_codes(orc):
    codes = np.arange(65536, dtype=np.uint16)
    mine = orc.bf16_to_f32(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_encode_matches_torch(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 10.0,
        rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.4e38, 1e-40, -1e-45], np.float32),
    ])
    x = x[~np.isnan(x)]
    mine = orc.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_e4m3_decode_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3_to_f32(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.nanmax(mine) == 448.0 and mine[1] == 2.0**-9


def _boundary_sweep():
    """Every fp32 within 64 ulps of each midpoint between neighbouring e4m3
    values, plus random patterns in [0, 464] and the subnormal range."""
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    vals = np.append(vals, 480.0)  # the value that would follow 448
    mids = ((vals[1:].astype(np.float64) + vals[:-1]) / 2).astype(np.float32)
    pts = [mids.view(np.int32)[:, None] + np.arange(-64, 65, dtype=np.int32)[None, :]]
    pts = np.concatenate([p.ravel() for p in pts]).view(np.float32)
    rng = np.random.default_rng(1)
    top = np.float32(464.0).view(np.int32)
    rand = rng.integers(0, top + 1, 3_000_000, dtype=np.int64).astype(np.int32).view(np.float32)
    sub = np.linspace(0, 2.0**-6, 100001, dtype=np.float32)
    x = np.concatenate([pts, rand, sub, vals[:-1]]).astype(np.float32)
    x = x[(x >= 0) & (x <= 464.0)]
    return np.concatenate([x, -x])


def test_e4m3_encode_matches_torch_rne():
    import oracle as orc

    x = _boundary_sweep()
    mine = orc.f32_to_e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(mine != ref)[0]
    assert bad.size == 0, (x[bad[:5]], mine[bad[:5]], ref[bad[:5]])


def test_e4m3_encode_saturates(orc):
    x = np.array([448.0, 464.0, 465.0, 1e6, np.inf, -1e6, -np.inf], np.float32)
    assert list(orc.f32_to_e4m3(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert orc.f32_to_e4m3(np.array([np.nan], np.float32))[0] == 0x7F


def test_f16_decode_all_codes(orc):
    codes = np.arange(65536, dtype=np.uint16)
    mine = orc.f16_to_f32(codes)
    ref = codes.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_encode_matches_numpy(orc):
    rng = np.random.default_rng(2)
    fin = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    mids = ((fin[1:].astype(np.float64) + fin[:-1]) / 2).astype(np.float32)
    near = (mids.view(np.int32)[:, None] + np.arange(-2, 3, dtype=np.int32)[None, :]).ravel()
    x = np.concatenate([near.view(np.float32), rng.standard_normal(500000).astype(np.float32) * 300,
                        rng.standard_normal(100000).astype(np.float32) * 1e-5])
    x = x[np.abs(x) < 65504.0]
    x = np.concatenate([x, -x])
    mine = orc.f32_to_f16(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)
    sat = orc.f32_to_f16(np.array([65504.0, 65520.0, 1e9, -1e9], np.float32))
    assert list(sat) == [0x7BFF, 0x7BFF, 0x7BFF, 0xFBFF]
