"""Pins of the oracle's number formats (OCP fp8 E4M3, MX e2m1 / E8M0, bf16)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import formats as of
from synth import formats as sf


def test_fp8_table_known_points():
    v = oracle.fp8_e4m3_values()
    assert v[0x00] == 0.0
    assert v[0x01] == 2.0 ** -9          # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert v[0x08] == 2.0 ** -6          # smallest normal
    assert v[0x38] == 1.0
    assert v[0x7E] == 448.0              # largest finite
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0xFE] == -448.0
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)      # codes 0..0x7E strictly increasing
    assert np.array_equal(v[0x80:0xFF], -pos)


def test_fp8_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.decode_fp8_e4m3(codes)
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.all(both_nan | (ref == ours))


def test_e2m1_and_e8m0():
    assert list(oracle.e2m1_values()[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(oracle.e2m1_values()[8:], -oracle.e2m1_values()[:8])
    d = oracle.decode_e8m0(np.array([0, 127, 128, 254, 255]))
    assert d[0] == 2.0 ** -127 and d[1] == 1.0 and d[2] == 2.0 and d[3] == 2.0 ** 127 and np.isnan(d[4])


def test_bf16_decode():
    x = np.array([1.0, -2.5, 3.140625, 65280.0], dtype=np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.decode_bf16(bits), x.astype(np.float64))


def test_bf16_encode_matches_torch_and_ties_to_even():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1e-40, -3e-39, 2.0 ** -126, 3.3895313892515355e38]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.encode_bf16(x.astype(np.float64)), ref)
    # exact midpoints between neighbours: 1 + 2^-8 lies between 1 and 1 + 2^-7 -> even significand (1.0);
    # 1 + 3*2^-8 lies between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> 1 + 2^-6
    mids = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -40])
    got = oracle.decode_bf16(oracle.encode_bf16(mids))
    assert list(got) == [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7]
    # a float64 value just above a float32 midpoint rounds up even where float32 would tie to even first
    v = 1 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.decode_bf16(oracle.encode_bf16(np.array([v])))[0] == 1 + 2.0 ** -7


def test_fp8_encoders_agree_and_match_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((300, 128)) * rng.uniform(0.01, 100, (300, 1))).astype(np.float32)
    c_syn, s_syn = sf.fp8_rowscale_encode(x)
    c_orc, s_orc = of.encode_fp8_rows(x.astype(np.float64))
    # scales: fp32 vs fp64 division of the same amax
    assert np.allclose(s_syn, s_orc, rtol=1e-6, atol=0)
    # codes: both round x/scale to nearest-even; allow only boundary ties from fp32 vs fp64 scale
    v = x.astype(np.float64) / s_orc[:, None]
    mism = c_syn != c_orc
    if mism.any():
        vals = oracle.fp8_e4m3_values()
        a = np.abs(v[mism])
        lo = np.abs(vals[c_orc[mism] & 0x7F])
        hi = np.abs(vals[c_syn[mism] & 0x7F])
        mid = 0.5 * (lo + hi)
        assert np.all(np.abs(a - mid) <= 1e-5 * mid)
    # torch's RNE cast of the same fp32 quotients
    q = (x / s_syn[:, None]).astype(np.float32)
    t = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(t, c_syn)


def test_fp8_saturation_and_ties():
    vals = np.array([500.0, 448.0, 460.0, -1e6, 2.0 ** -10, 3 * 2.0 ** -10, 1.0625, 1.1875], np.float32)
    codes = sf.fp8_e4m3_encode(vals)
    dec = oracle.decode_fp8_e4m3(codes)
    # 2^-10 is halfway between 0 and 2^-9 -> even code 0; 3*2^-10 is halfway 2^-9 / 2*2^-9 -> even (2*2^-9)
    assert list(dec) == [448.0, 448.0, 448.0, -448.0, 0.0, 2 * 2.0 ** -9, 1.0, 1.25]


def test_mxfp4_round_trip_bound_and_encoders_agree():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    p1, e1 = sf.mxfp4_encode(x)
    p2, e2 = of.encode_mxfp4(x.astype(np.float64))
    assert np.array_equal(e1, e2)
    assert np.array_equal(p1, p2)
    xr = oracle.decode_mxfp4(p1, e1)
    blk_scale = np.repeat(oracle.decode_e8m0(e1), 32, axis=-1)
    v = x / blk_scale
    err = np.abs(xr - x) / blk_scale
    # spacing of e2m1 is 0.5 below 2, 1 in [2, 4], 2 in [4, 6]; beyond 6 saturates
    bound = np.where(np.abs(v) <= 2, 0.25, np.where(np.abs(v) <= 4, 0.5, 1.0))
    sat = np.abs(v) > 6
    assert np.all((err <= bound + 1e-12) | sat)
    assert np.all(np.abs(xr[sat]) == 6 * blk_scale[sat])
    # shared exponent: amax / 2^X lies in [4, 8)
    amax = np.abs(x.reshape(64, 4, 32)).max(-1)
    r = amax / oracle.decode_e8m0(e1)
    assert np.all((r >= 4) & (r < 8))


@pytest.mark.parametrize("v,expect", [(0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0),
                                      (3.5, 4.0), (5.0, 4.0), (7.0, 6.0), (-0.3, -0.5)])
def test_e2m1_ties_to_even(v, expect):
    code = sf.e2m1_encode(np.array([v]))
    assert oracle.decode_e2m1(code)[0] == expect


def test_fp8_rope_rows_layout_and_values():
    """The mixed KV row: c - R e4m3 codes of value/scale (scale = amax/448 of those values), then the R
    RoPE values as little-endian bf16.  A hand-built row: the largest fp8-part value maps to code 0x7E
    (448), a value of a quarter of it to 0x6E (112), a negative one to the sign bit set, zero to 0."""
    c, R = 32, 16
    x = np.zeros((1, c))
    x[0, 0] = 3.5            # amax: scale = 3.5 / 448
    x[0, 1] = 3.5 / 4        # 112 * scale
    x[0, 2] = -3.5 / 4
    x[0, 16] = 1.0           # RoPE part: bf16 1.0 = 0x3F80
    x[0, 31] = -2.5          # 0xC020
    data, scale = oracle.encode_fp8_rope_rows(x, R)
    assert data.shape == (1, c + R) and data.dtype == np.uint8
    assert scale[0] == 3.5 / 448
    assert list(data[0, :4]) == [0x7E, 0x6E, 0xEE, 0x00]
    bf = data[0, c - R:].view(np.uint16)
    assert bf[0] == 0x3F80 and bf[15] == 0xC020 and np.all(bf[1:15] == 0)
    back = oracle.decode_fp8_rope_rows(data, scale, R)
    assert np.array_equal(back, x)


def test_fp8_rope_rows_round_trip_bound():
    """Decoded values: RoPE dims within bf16 rounding (2^-8 relative), the others within half an e4m3
    step of their scaled value (at most 2^-4 relative above 2^-6 * scale, 2^-10 * scale absolute below)."""
    r = np.random.default_rng(3)
    x = r.standard_normal((50, 512))
    data, scale = oracle.encode_fp8_rope_rows(x, 64)
    back = oracle.decode_fp8_rope_rows(data, scale, 64)
    fp, rp = x[:, :448], x[:, 448:]
    assert np.all(np.abs(back[:, 448:] - rp) <= np.abs(rp) * 2.0 ** -8)
    err = np.abs(back[:, :448] - fp)
    s = scale[:, None]
    assert np.all(err <= np.maximum(np.abs(fp) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-12))
    # the largest fp8-part value comes back as 448 times the scale, stored in float32
    assert np.allclose(np.max(np.abs(back[:, :448]), axis=1), np.max(np.abs(fp), axis=1), rtol=2e-7)
