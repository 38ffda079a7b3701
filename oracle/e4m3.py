"""OCP OFP8 E4M3 codec.  Test infrastructure: see the package docstring.

The pages fix the format only through its range: page "FP8量化在生成式推荐系统
OneRec-V2中的优化实践", §1.2, puts activations inside the FP8 interval +/-448, and
§2.2 names E4M3 (4 exponent bits, 3 mantissa bits) for weights.  +/-448 as the
largest finite value is the OCP "OFP8" E4M3 variant (bias 7, no infinities, a single
NaN mantissa pattern), which is what this module implements.

Byte layout ``s eeee mmm``:

* ``e == 0``            -> (-1)^s * m * 2^-9                (subnormals, +/-0 at m == 0)
* ``1 <= e <= 15``      -> (-1)^s * (8 + m) * 2^(e - 10)     (normals)
* ``e == 15, m == 7``   -> NaN (bytes 0x7F and 0xFF).  There is no infinity.

Encoding (``encode``) is the saturating cast used by the quantizer: NaN stays NaN,
magnitudes at or above 448 (including infinities) become +/-448, everything else is
rounded to the nearest representable magnitude with ties to even, and the sign is
kept (so -0 and negative underflow give 0x80).
"""

import numpy as np

MAX_FINITE = 448.0
MIN_NORMAL = 2.0 ** -6
MIN_SUBNORMAL = 2.0 ** -9
BIAS = 7
NAN_CODES = (0x7F, 0xFF)


def decode(codes):
    """E4M3 bytes -> float64 values (NaN for 0x7F / 0xFF), elementwise."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    neg = (c >> 7) == 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    subnormal = m * MIN_SUBNORMAL
    normal = (8 + m) * np.exp2((e - 10).astype(np.float64))
    mag = np.where(e == 0, subnormal, normal)
    val = np.where(neg, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def encode(values):
    """float64 values -> E4M3 bytes: saturate to +/-448, round to nearest even, keep sign.

    The input is taken exactly as given (the quantizer hands in values that are
    already FP32-rounded).  Scaling by powers of two is exact in float64 and
    ``np.rint`` rounds half to even, so every step below is exact.
    """
    v = np.asarray(values, dtype=np.float64)
    neg = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int64)

    is_nan = np.isnan(a)
    is_sat = ~is_nan & (a >= MAX_FINITE)
    is_sub = ~is_nan & ~is_sat & (a < MIN_NORMAL)
    is_nrm = ~is_nan & ~is_sat & ~is_sub

    # Below the smallest normal the spacing is fixed at 2^-9.  A result of 8 units is
    # the smallest normal, whose byte is also 8 (e = 1, m = 0), so the carry needs no
    # special case.
    code[is_sub] = np.rint(a[is_sub] / MIN_SUBNORMAL).astype(np.int64)

    # Normals: binade exponent E = floor(log2 a), spacing 2^(E-3), significand
    # n = a / spacing in [8, 16].  Rounding up to 16 carries into the next binade.
    an = a[is_nrm]
    _, fexp = np.frexp(an)  # an = f * 2^fexp with f in [0.5, 1)
    E = fexp.astype(np.int64) - 1
    n = np.rint(an / np.exp2((E - 3).astype(np.float64))).astype(np.int64)
    carry = n == 16
    E = np.where(carry, E + 1, E)
    n = np.where(carry, 8, n)
    code[is_nrm] = ((E + BIAS) << 3) | (n - 8)

    code[is_sat] = 0x7E
    code[is_nan] = 0x7F
    return (code | (neg << 7)).astype(np.uint8)


def table():
    """The 256 decoded values, indexed by byte."""
    return decode(np.arange(256, dtype=np.uint8))
