"""Pins of the oracle's E4M3 codec (CPU only)."""

import numpy as np
import pytest

from oracle import e4m3_decode, e4m3_encode
from tests import pins


def test_decode_closed_form_points():
    # OCP OFP8 E4M3: max normal S.1111.110 = 1.75 * 2**8, min normal
    # S.0001.000 = 2**-6, max subnormal S.0000.111 = 0.875 * 2**-6, min
    # subnormal S.0000.001 = 2**-9, one = S.0111.000.
    d = e4m3_decode(np.array([0x7E, 0xFE, 0x08, 0x07, 0x01, 0x38, 0x40, 0x30, 0x78, 0x3C],
                             dtype=np.uint8))
    assert list(d) == [1.75 * 2 ** 8, -1.75 * 2 ** 8, 2.0 ** -6, 0.875 * 2 ** -6, 2.0 ** -9,
                       1.0, 2.0, 0.5, 256.0, 1.5]
    z = e4m3_decode(np.array([0x00, 0x80], dtype=np.uint8))
    assert z[0] == 0 and z[1] == 0 and not np.signbit(z[0]) and np.signbit(z[1])
    n = e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))
    assert np.isnan(n).all()


def test_decode_all_codes_match_torch_float8_e4m3fn():
    assert pins.check_decode_against_torch(e4m3_decode)


def test_decode_structure():
    v = e4m3_decode(np.arange(256, dtype=np.uint8))
    pos = v[:0x7F]
    # non-negative codes 0x00..0x7E are strictly increasing
    assert np.all(np.diff(pos) > 0)
    # negative half mirrors the positive half
    assert np.array_equal(v[0x80:0xFF], -pos)
    finite = v[~np.isnan(v)]
    assert len(np.unique(finite)) == 253  # +0 and -0 compare equal
    # every value is exact in fp16 (the conversion used on the device is lossless)
    assert np.array_equal(finite.astype(np.float16).astype(np.float64), finite)


def test_encode_round_trip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), codes)


def test_encode_saturation_and_specials():
    x = np.array([448.0, 449.0, 464.0, 480.0, 1e6, np.inf, -448.0, -500.0, -np.inf], dtype=np.float32)
    assert list(e4m3_encode(x)) == [0x7E] * 6 + [0xFE] * 3
    nan = e4m3_encode(np.array([np.nan, -np.nan], dtype=np.float32))
    assert (nan & 0x7F).tolist() == [0x7F, 0x7F]
    # signed zero and values below half the smallest subnormal
    tiny = np.array([0.0, -0.0, 2.0 ** -11, -2.0 ** -11, 2.0 ** -10, 3 * 2.0 ** -10], dtype=np.float32)
    assert list(e4m3_encode(tiny)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x02]


def test_encode_midpoints_and_neighbours():
    # every midpoint between adjacent positive codes, and one fp32 ulp either side
    vals = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    for arr in (mids, up, dn, -mids, -up, -dn):
        assert np.array_equal(e4m3_encode(arr), pins.brute_force_encode(arr))
    lower = np.arange(0x7E, dtype=np.int64)
    # at a tie the even code wins
    got = e4m3_encode(mids).astype(np.int64)
    assert np.all(got % 2 == 0)
    assert np.all((got == lower) | (got == lower + 1))


def test_encode_brute_force_all_fp16_inputs_several_scales():
    bits = np.arange(65536, dtype=np.uint16)
    x = bits.view(np.float16)
    x = x[np.isfinite(x)].astype(np.float32)
    for scale in (np.float32(1.0), np.float32(0.0123), np.float32(1 / 448), np.float32(3.7)):
        q = (x.astype(np.float64) / np.float64(scale)).astype(np.float32)
        assert np.array_equal(e4m3_encode(q), pins.brute_force_encode(q)), scale


def test_encode_random_fp32_matches_torch_clamped():
    rng = np.random.default_rng(1234)
    # spread over many binades, both signs, including the subnormal range and overflow
    mant = rng.uniform(1.0, 2.0, 2_000_000)
    expo = rng.integers(-14, 12, 2_000_000)
    sign = rng.choice([-1.0, 1.0], 2_000_000)
    x = (sign * mant * np.exp2(expo)).astype(np.float32)
    assert np.array_equal(e4m3_encode(x), pins.torch_encode_clamped(x))


def test_encode_random_fp32_matches_brute_force():
    rng = np.random.default_rng(99)
    x = (rng.standard_normal(300_000) * np.exp2(rng.integers(-12, 10, 300_000))).astype(np.float32)
    assert np.array_equal(e4m3_encode(x), pins.brute_force_encode(x))


@pytest.mark.parametrize("mistake", ["bias8", "truncate", "no_saturate", "fnuz_nan"])
def test_pins_catch_planted_codec_mistakes(mistake):
    """Plant a plausible mistake in a copy of the codec and check a pin fails."""
    def decode_bad(c):
        c = np.asarray(c, np.uint8).astype(np.int64)
        s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
        if mistake == "bias8":
            mag = np.where(e == 0, m * 2.0 ** -10, (1 + m / 8) * np.exp2(e - 8.0))
        else:
            mag = np.where(e == 0, m * 2.0 ** -9, (1 + m / 8) * np.exp2(e - 7.0))
        val = np.where(s == 1, -mag, mag)
        if mistake == "fnuz_nan":
            return np.where(c == 0x80, np.nan, val)
        return np.where((e == 15) & (m == 7), np.nan, val)

    def encode_bad(x):
        v = np.asarray(x, np.float32)
        if mistake == "truncate":
            # truncation toward zero instead of nearest-even
            vals = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
            a = np.abs(v.astype(np.float64))
            idx = np.searchsorted(vals, a, side="right") - 1
            idx = np.clip(idx, 0, 0x7E)
            return (idx | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)
        if mistake == "no_saturate":
            out = e4m3_encode(v)
            return np.where(np.abs(v) > 464, 0x7F | (out & 0x80), out).astype(np.uint8)
        return e4m3_encode(v)

    caught = not pins.check_decode_against_torch(decode_bad)
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(50_000) * 200).astype(np.float32)
    caught |= not np.array_equal(encode_bad(x), pins.brute_force_encode(x))
    assert caught
