"""Pins of the oracle's number formats against library casts and closed forms.

OCP e4m3fn (the fp8 of the weight/activation blocks, SGLang-H20 report,
Prefill solutions: MoE b_scale handling) and bfloat16 rounding.
"""
import numpy as np
import pytest
import torch


def test_e4m3_decode_all_codes_match_torch(orc):
    codes = np.arange(256, dtype=np.uint8)
    mine = orc.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2  # 0x7f and 0xff
    assert np.array_equal(mine[~nan], ref[~nan])
    assert mine[0x7e] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def _torch_e4m3(v):
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_every_bf16_in_range_matches_torch(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint32) << 16
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 464.0)]  # torch turns larger values into NaN
    assert np.array_equal(orc.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_encode_random_fp32_and_ties(orc):
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 50,
        rng.standard_normal(50_000).astype(np.float32) * 1e-2,
        rng.uniform(-2e-3, 2e-3, 50_000).astype(np.float32),   # subnormal range
    ])
    # exact midpoints between neighbouring codes: ties go to the even code
    grid = orc.e4m3_decode(np.arange(0, 0x7e, dtype=np.uint8)).astype(np.float64)
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids]).astype(np.float32)
    v = v[np.abs(v) <= 464.0]
    mine = orc.e4m3_encode(v)
    assert np.array_equal(mine, _torch_e4m3(v))
    tie_codes = orc.e4m3_encode(mids)
    assert np.all(tie_codes % 2 == 0)


def test_e4m3_encode_saturates(orc):
    v = np.array([448.0, 463.9, 464.0, 1e6, -1e30, np.float32(3.4e38)], np.float32)
    assert list(orc.e4m3_encode(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E]


def test_bf16_round_matches_torch_on_fp32_inputs(orc):
    rng = np.random.default_rng(3)
    f = np.concatenate([rng.standard_normal(100_000) * 10.0 ** rng.integers(-30, 30, 100_000),
                        (np.arange(1, 2000) * 2.0 ** -140)]).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.bf16_round(f.astype(np.float64)), ref)


def test_bf16_round_is_nearest_for_doubles(orc):
    """Single rounding of a double: no representable bf16 is closer (ties even)."""
    rng = np.random.default_rng(4)
    d = rng.standard_normal(20_000) * 3.0
    u = orc.bf16_round(d).astype(np.int64)
    here = orc.bf16_to_f32(u.astype(np.uint16)).astype(np.float64)
    up = orc.bf16_to_f32((u + 1).astype(np.uint16)).astype(np.float64)
    dn = orc.bf16_to_f32((u - 1).astype(np.uint16)).astype(np.float64)
    err = np.abs(here - d)
    assert np.all(err <= np.abs(up - d)) and np.all(err <= np.abs(dn - d))
    # a value just above a bf16 tie must round up (a float detour would lose it)
    assert orc.bf16_round(np.array([1.0 + 2 ** -8 + 2 ** -30]))[0] == 0x3F81


def test_quantize_1x128_closed_form(orc):
    rng = np.random.default_rng(11)
    v = (rng.standard_normal((5, 512)) * rng.uniform(1e-3, 10, (5, 1))).astype(np.float32)
    v[2, 128:256] = 0.0  # an all-zero block
    codes, scales = orc.quantize_1x128(v)
    assert codes.shape == (5, 512) and scales.shape == (5, 4)
    blocks = v.reshape(5, 4, 128)
    amax = np.abs(blocks).max(axis=2)
    expect = np.where(amax == 0, np.float32(1), (amax / np.float32(448)).astype(np.float32))
    assert np.array_equal(scales, expect)
    assert np.all(codes[2, 128:256] == 0)
    dq = orc.e4m3_decode(codes).reshape(5, 4, 128).astype(np.float64) * scales[:, :, None]
    # the block's largest magnitude lands on +-448 and every value within half an e4m3 step
    for r in range(5):
        for b in range(4):
            if amax[r, b] == 0:
                continue
            i = np.abs(blocks[r, b]).argmax()
            assert codes[r, b * 128 + i] & 0x7F == 0x7E
            x = blocks[r, b].astype(np.float64)
            step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(x / scales[r, b]), 2 ** -6))) - 3), 2 ** -9)
            assert np.all(np.abs(dq[r, b] - x) <= 0.5 * step * scales[r, b] * (1 + 1e-6))
    # codes equal torch's e4m3 cast of the fp32 quotient
    q = (blocks / scales[:, :, None]).astype(np.float32).clip(-448, 448).reshape(5, 512)
    assert np.array_equal(codes, _torch_e4m3(q))
