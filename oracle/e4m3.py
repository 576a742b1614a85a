"""E4M3 codec, float64 reference.

Decode follows the closed form of the OCP 8-bit floating point specification
(OFP8), E4M3 variant: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits, no infinities, the all-ones exponent with all-ones mantissa is NaN,
largest finite magnitude 448.

The pages fix only that the cache is E4M3 and that the decoder is exact
("Integrate calibrated E4M3 QSA KV capacity path", Changes: the decoder is a
bit-exact software decode). Encoding is not described on the pages; the
readings used here are: round to nearest with ties to even, magnitudes at or
above 448 (including infinity) saturate to +-448, NaN maps to a NaN code with
its sign, and the sign of zero is kept.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code as float64 (NaN for 0x7F and 0xFF).

    For code c with sign s = c >> 7, exponent field e = (c >> 3) & 15 and
    mantissa m = c & 7: e == 0 gives the subnormal m * 2**-9, otherwise the
    value is (1 + m / 8) * 2**(e - 7); the sign bit negates (so 0x80 is -0).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    magnitude = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    value = np.where(s == 1, -magnitude, magnitude)
    return np.where((e == 15) & (m == 7), np.nan, value)


def e4m3_encode(x) -> np.ndarray:
    """Saturating round-to-nearest-even E4M3 code of each float32 value.

    Steps (all exact in float64 because every scaling is a power of two):

    1. NaN -> 0x7F with the input's sign bit.
    2. |x| >= 448 (and +-inf) -> 0x7E with the sign (saturation).
    3. |x| < 2**-6 (below the smallest normal): k = RNE(|x| * 2**9) is the
       code magnitude directly; k == 8 lands exactly on the smallest normal.
    4. otherwise, with e = floor(log2 |x|): k = RNE(|x| / 2**(e - 3)) lies in
       [8, 16]; k == 16 carries into the next binade (e + 1, k = 8); the code
       magnitude is (e + 7) << 3 | (k - 8).
    5. the sign bit is ORed in, so a negative value rounding to zero gives 0x80.
    """
    v = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    a = np.abs(v)
    code = np.zeros(v.shape, dtype=np.int64)
    nan = np.isnan(a)
    sat = ~nan & (a >= E4M3_MAX)
    sub = ~nan & (a < 2.0 ** -6)
    nrm = ~nan & ~sat & ~sub

    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)

    an = a[nrm]
    _, ex = np.frexp(an)  # an = f * 2**ex with f in [0.5, 1)
    e = ex.astype(np.int64) - 1
    k = np.rint(an / np.exp2(e - 3.0)).astype(np.int64)
    carry = k == 16
    e = np.where(carry, e + 1, e)
    k = np.where(carry, 8, k)
    code[nrm] = ((e + 7) << 3) | (k - 8)

    code[sat] = 0x7E
    code[nan] = 0x7F
    return (code | sign).astype(np.uint8)
