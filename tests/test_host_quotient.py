"""The quotient the cache write encodes, CPU only.

The write's code is E4M3(fl32(x) / scale) with the quotient rounded once to
fp32. The grouped write kernel does not divide: it multiplies x (an fp16
value) by 1 / scale rounded to fp64 and rounds that product to fp32. That is
the same fp32 value for any fp32 x and normal fp32 scale with a quotient in
the fp32 normal range, because x / scale then lies more than 2^-49 (relative)
away from every fp32 rounding midpoint while the fp64 product is within about
2^-52 of it. These tests check the claim with IEEE arithmetic in numpy: every
finite fp16 value against scales over many binades, including significands at
the ends of their range, fp32 inputs, and fp64 division rounded to fp32."""
import numpy as np
import pytest

ALL_F16 = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
ALL_F16 = ALL_F16[np.isfinite(ALL_F16)]


def scales(seed, n):
    rng = np.random.default_rng(seed)
    sig = np.concatenate([rng.integers(1 << 23, 1 << 24, n),
                          [(1 << 24) - 1, (1 << 24) - 2, (1 << 24) - 3, (1 << 23) + 1, (1 << 23) + 3, 1 << 23,
                           0xAAAAAA, 0xD55555, 0xC00001, 0xFFFFF1]])
    exps = rng.integers(-40, 40, sig.size)
    s = (sig.astype(np.float64) * 2.0 ** (exps - 23)).astype(np.float32)
    extra = np.float32([1.0, 448.0, 1 / 448.0, 3.0, 7.0, 0.1, 1e-6, 1e6, np.float32(2.0 ** -126) * 3])
    return np.concatenate([s, extra])


def via_reciprocal(x16, scale):
    return (x16.astype(np.float64) * (1.0 / np.float64(scale))).astype(np.float32)


@pytest.mark.parametrize("seed", range(4))
def test_reciprocal_product_equals_fp32_division(seed):
    x32 = ALL_F16.astype(np.float32)
    bad = []
    with np.errstate(over="ignore", under="ignore"):
        for s in scales(100 + seed, 250):
            ref = x32 / np.float32(s)
            got = via_reciprocal(ALL_F16, s)
            n = int(np.sum(ref.view(np.uint32) != got.view(np.uint32)))
            if n:
                bad.append((float(s), n))
    assert not bad, bad[:5]


def test_fp64_division_rounded_to_fp32_agrees_too():
    # the oracle's calibration divides in fp64 and rounds once (innocuous
    # double rounding); the same holds for this quotient
    x32 = ALL_F16.astype(np.float32)
    with np.errstate(over="ignore", under="ignore"):
        for s in scales(7, 60):
            ref = x32 / np.float32(s)
            got = (ALL_F16.astype(np.float64) / np.float64(s)).astype(np.float32)
            assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), float(s)


def test_fp32_inputs_agree_as_well():
    # the argument needs only that x's significand (24 bits at most) is
    # narrower than a midpoint's odd significand (25 bits): fp32 inputs too
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(1_000_000), rng.uniform(-1e4, 1e4, 1_000_000)]).astype(np.float32)
    with np.errstate(over="ignore", under="ignore"):
        for s in scales(11, 8):
            ref = x / np.float32(s)
            got = (x.astype(np.float64) * (1.0 / np.float64(s))).astype(np.float32)
            assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), float(s)
