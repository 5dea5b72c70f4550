"""Pins of the oracle's number formats against torch's own codecs.

bf16 and OCP E4M3 ("e4m3fn") decoding is pinned code by code; the e4m3
encoder (round to nearest, ties to even, saturating at +-448) is pinned at
every representable value, every midpoint and one fp32 ulp either side of
it; the per-row activation quantisation rule is pinned by closed-form rows
and by torch's cast.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def test_bf16_table_matches_torch_all_codes():
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_value(c) for c in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros and infinities keep their sign
    assert math.copysign(1.0, got[0x8000]) == -1.0
    assert got[0x7F80] == math.inf and got[0xFF80] == -math.inf


def test_e4m3_table_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(got), nan)   # 0x7F and 0xFF only
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def _positive_finite():
    return np.array([oracle.e4m3_value(c) for c in range(127)])


def _torch_e4m3(v):
    return torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encoder_representable_values_round_trip():
    vals = _positive_finite()
    for c, v in enumerate(vals):
        assert oracle.e4m3_encode(v) == c
        assert oracle.e4m3_encode(-v) == (0x80 | c)


def test_encoder_midpoints_and_neighbours_match_torch():
    vals = _positive_finite()
    mids = (vals[:-1] + vals[1:]) / 2           # exact in fp32 (short mantissas)
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)
    probes = np.concatenate([mids32,
                             np.nextafter(mids32, np.float32(np.inf)),
                             np.nextafter(mids32, np.float32(0))]).astype(np.float32)
    probes = np.concatenate([probes, -probes])
    got = oracle.e4m3_encode_array(probes)
    ref = _torch_e4m3(probes)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("v,code", [
    (17.0, 0x58),            # tie between 16 and 18 -> 16 (even mantissa)
    (19.0, 0x5A),            # tie between 18 and 20 -> 20
    (2.0 ** -10, 0x00),      # half the smallest subnormal -> 0
    (1.5 * 2.0 ** -9, 0x02),  # tie between 1 and 2 quanta -> 2 quanta
    (0.75 * 2.0 ** -9, 0x01),  # above the half quantum -> smallest subnormal
    (7.5 * 2.0 ** -9, 0x08),  # tie at the subnormal/normal boundary -> 2^-6
])
def test_encoder_hand_cases(v, code):
    assert oracle.e4m3_encode(v) == code
    assert _torch_e4m3([v])[0] == code


def test_encoder_saturates_and_nan():
    for v in [448.0, 448.5, 463.9, 464.0, 479.0, 480.0, 1e6, 3.0e38, math.inf]:
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE
    assert oracle.e4m3_encode(math.nan) == 0x7F
    # below 464 torch agrees (it only differs by giving NaN from 480 up)
    assert _torch_e4m3([448.5, 463.9])[0] == 0x7E


def test_encoder_random_values_match_torch():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-9, 6, 20000))).astype(np.float32)
    v = v[np.abs(v) < 448]
    assert np.array_equal(oracle.e4m3_encode_array(v), _torch_e4m3(v))


def test_encoder_signed_zero_and_underflow():
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-30) == 0x80
    assert _torch_e4m3([-1e-30])[0] == 0x80


def test_quant_row_zero_row():
    codes, s = oracle.quant_row(np.zeros(33, dtype=np.float32))
    assert s == 1.0 and not codes.any()


def test_quant_row_exact_448_row_is_identity():
    # amax = 448 gives scale 1 and inv 1: codes are the plain encodings
    vals = _positive_finite()
    row = np.concatenate([vals[::5], -vals[::7], [448.0]]).astype(np.float32)
    codes, s = oracle.quant_row(row)
    assert s == 1.0
    assert np.array_equal(codes, _torch_e4m3(row))
    assert np.array_equal([oracle.e4m3_value(c) for c in codes], row.astype(np.float64))


def test_quant_row_power_of_two_amax():
    # amax = 7 * 2^-3 = 0.875: scale = 0.875/448 = 2^-9 exactly, inv = 512
    row = np.array([0.875, -0.5, 0.25, 0.001, -0.875], dtype=np.float32)
    codes, s = oracle.quant_row(row)
    assert s == 2.0 ** -9
    assert np.array_equal(codes, _torch_e4m3(row * np.float32(512.0)))
    assert oracle.e4m3_value(codes[0]) == 448.0 and oracle.e4m3_value(codes[4]) == -448.0


def _torch_quant_rows(x32):
    amax = x32.abs().amax(dim=1)
    s = torch.where(amax > 0, (amax.double() / 448.0).float(), torch.ones_like(amax))
    inv = torch.where(amax > 0, (448.0 / amax.double()).float(), torch.ones_like(amax))
    q = (x32 * inv[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.numpy(), s.numpy()


def test_quant_rows_bf16_matches_torch_cast():
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(37, 300, generator=g) * 3).to(torch.bfloat16)
    x[5] = 0
    x[7, :] = 0
    x[7, 11] = -2.5
    codes, scales = oracle.quant_rows_bf16(x)
    rq, rs = _torch_quant_rows(x.float())
    assert np.array_equal(scales, rs)
    assert np.array_equal(codes, rq)
    assert scales[5] == 1.0 and not codes[5].any()
    assert oracle.e4m3_value(codes[7, 11]) == -448.0
